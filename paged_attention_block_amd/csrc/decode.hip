// Grouped-query paged decode for bf16 caches on gfx950: split-K chunks + log-sum-exp merge.
//
// The operation (MinivLLM API docs, "Attention", paged_attention_decode): one query per
// sequence, attending its seq_lens[s] cached keys through the block table, online softmax.
// Long contexts are split over the key axis (vLLM learning book section 7: split-KV wins
// small-batch long-sequence decode); each piece leaves (m, l, O) and a merge rescales them
// by exp2(m_p - max m).
//
// Work item = one wavefront per (chunk of the batch's key steps, KV head g).  All G query
// heads of the group share every K/V row the wave streams, so each KV byte is read from HBM
// once.
// The math runs on MFMA even though decode is bandwidth-bound: at G = 8 the plain-FMA
// version needs ~4 FMAs per cache byte, more than the vector ALU can retire at 8 TB/s.
//
// Lane layout (v_mfma_f32_16x16x32_bf16, lane l: col = l % 16, grp = l / 16):
//   S^T = K . Q^T   A = K rows (m = key col, k = 8 dims of 32-dim slice t at 8*grp),
//                   B = Q^T (n = head col), C: lane holds keys 4*grp + r of the 16-key
//                   group for head col.
//   O^T = V^T . P^T A = V^T (m = dim, k = keys), B = P^T straight from the S^T accumulator
//                   registers (keys 16a + 4*grp + r, a = 0, 1, are the 8 k-values of lane
//                   group grp).  The V rows are loaded 16 B per lane (8 dims of one key),
//                   8 keys per lane, and transposed in registers with byte permutes: PV
//                   MFMA t then covers dims d = DPL*m + t, m = 0..15.
//   The output C of PV MFMA t holds, in lane l, dims DPL*(4*grp + r) + t for head col:
//   each lane owns DPL*4 consecutive dims of one head.
#include <math.h>

#include <atomic>

#include "pa_internal.hpp"

namespace pa {

namespace {

__device__ inline uint32_t pack_bf16(float lo, float hi) { return pack_bf16x2(lo, hi); }

// DPL = dims per lane chunk of a V row: 8 (16 B) for D = 128, 4 (8 B) for D = 64.
template <int D> struct VRow;
template <> struct VRow<128> { typedef u32x4 T; };
template <> struct VRow<64> { typedef u32x2 T; };
// the same V piece in an FP8 cache: DPL bytes
template <int D> struct VRow8;
template <> struct VRow8<128> { typedef u32x2 T; };
template <> struct VRow8<64> { typedef uint32_t T; };

// Two FP8 (E4M3) cache bytes -> two bf16, exactly (every E4M3 value is a bf16 value).
__device__ inline uint32_t e4m3x2_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false));
}
__device__ inline uint32_t e4m3x2_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true));
}

}  // namespace

// Register types of one 32-key step as loaded: bf16 rows, or FP8 rows at half the bytes
// (widened to bf16 right before the step's MFMAs).  K: k[2][D/32], V: v[8].
template <int D, bool FP8> struct StepT;
template <int D> struct StepT<D, false> {
    typedef u32x4 K;
    typedef typename VRow<D>::T V;
};
template <int D> struct StepT<D, true> {
    typedef u32x2 K;
    typedef typename VRow8<D>::T V;
};

// Per-lane byte offsets from a 16-key group's first row: K rows (key col, 16 bytes at 16*grp
// of each 32-dim (bf16) or 64-dim (FP8) piece), V rows (key 4*grp + j%4, dims DPL*col).
//
// K.Q^T sums over the dims in any order as long as q uses the same one, so the MFMA k-slices
// need not be 32 consecutive dims.  bf16: slice t = dims 32t + 8*grp .. +8 (one 16-byte load).
// FP8: one 16-byte load brings dims 64u + 16*grp .. +16, split into slices t = 2u (first 8)
// and 2u + 1 (last 8): half the K load instructions of 8-byte loads.  q_slice() gives the
// matching 16-byte piece of the bf16 q row for slice t.
template <int D, bool FP8>
__device__ inline void lane_offsets(int col, int grp, uint32_t row_bytes, uint32_t& k_off, uint32_t& v_off) {
    constexpr int ELT = FP8 ? 1 : 2;
    k_off = (uint32_t)col * row_bytes + 16u * grp;
    v_off = (uint32_t)(4 * grp) * row_bytes + (uint32_t)(ELT * (D / 16)) * col;
}
template <bool FP8>
__device__ inline int q_slice(int t, int grp) { return FP8 ? 8 * (t >> 1) + 2 * grp + (t & 1) : 4 * t + grp; }

// Block-table rows are read through the constant address space.  The table is never written
// during a call, but the compiler cannot prove that of a plain pointer once the kernel stores
// its outputs, and then reads it with vector loads: a step's table lookup then waits for every
// load in flight (the wait counts are in order), including the other register set's, which
// leaves one step loading at a time.  Read as constant memory, the lookups are scalar loads,
// counted apart from the vector loads.
typedef const __attribute__((address_space(4))) int32_t* const_table_t;

// Loads of the 32-key step at k0 into registers: K rows (2 groups of 16 keys x KS slices,
// MFMA A-operand layout) and the V rows one lane needs for the PV MFMAs (8 keys x DPL
// dims).  Both 16-key groups of a step lie in one physical block each (block_size >= 16,
// 16-aligned); a group with no live key is never looked up and its lanes read the other
// group's rows instead, so every load is in bounds and unconditional.  Keys outside
// [kb, ke) are masked after the load.
template <int D, bool FP8>
__device__ __forceinline__ void load_step(int k0, int kb, int ke, const_table_t table,
                                          int shift, int BS, int64_t row_elems, int g,
                                          const char* __restrict__ kplane,
                                          const char* __restrict__ vplane, uint32_t k_off,
                                          uint32_t v_off, uint32_t row_bytes,
                                          typename StepT<D, FP8>::K (&kr)[2][D / 32],
                                          typename StepT<D, FP8>::V (&vr)[8]) {
    constexpr int ELT = FP8 ? 1 : 2;
    // wave-uniform byte offset of (first key of each 16-key group, KV head g) in a plane
    int64_t gb[2];
    bool gv[2];
#pragma unroll
    for (int ga = 0; ga < 2; ++ga) {
        const int j0 = k0 + 16 * ga;
        gv[ga] = (j0 < ke) && (j0 + 16 > kb);
        const int blk = gv[ga] ? table[j0 >> shift] : 0;
        gb[ga] = (((int64_t)blk * BS + (j0 & (BS - 1))) * row_elems + (int64_t)g * D) * ELT;
    }
    if (!gv[0]) gb[0] = gb[1];
    if (!gv[1]) gb[1] = gb[0];
#pragma unroll
    for (int ga = 0; ga < 2; ++ga) {
        const char* base = kplane + gb[ga];
        if constexpr (FP8) {
#pragma unroll
            for (int u = 0; u < D / 64; ++u) {
                const u32x4 x = *(const u32x4*)(base + k_off + 64 * u);
                kr[ga][2 * u] = u32x2{x[0], x[1]};
                kr[ga][2 * u + 1] = u32x2{x[2], x[3]};
            }
        } else {
#pragma unroll
            for (int t = 0; t < D / 32; ++t) kr[ga][t] = *(const u32x4*)(base + k_off + 64 * t);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const char* base = vplane + gb[j >> 2] + (int64_t)(j & 3) * row_bytes;
        vr[j] = *(const typename StepT<D, FP8>::V*)(base + v_off);
    }
}

// load_step for the step holding a sequence's new token (key kn) when the store is fused: the
// lanes whose K or V row is that key read it from the caller's row (knew_row / vnew_row: KV head
// g's D elements) instead of the cache slot, which the store has not written yet.  bf16 only.
template <int D>
__device__ __forceinline__ void load_step_new(int k0, int kb, int ke, const_table_t table,
                                              int shift, int BS, int64_t row_elems, int g,
                                              const char* __restrict__ kplane,
                                              const char* __restrict__ vplane, uint32_t k_off,
                                              uint32_t v_off, uint32_t row_bytes, int col, int grp, int kn,
                                              const char* knew_row, const char* vnew_row,
                                              u32x4 (&kr)[2][D / 32], typename VRow<D>::T (&vr)[8]) {
    int64_t gb[2];
    bool gv[2];
#pragma unroll
    for (int ga = 0; ga < 2; ++ga) {
        const int j0 = k0 + 16 * ga;
        gv[ga] = (j0 < ke) && (j0 + 16 > kb);
        const int blk = gv[ga] ? table[j0 >> shift] : 0;
        gb[ga] = (((int64_t)blk * BS + (j0 & (BS - 1))) * row_elems + (int64_t)g * D) * 2;
    }
    if (!gv[0]) gb[0] = gb[1];
    if (!gv[1]) gb[1] = gb[0];
#pragma unroll
    for (int ga = 0; ga < 2; ++ga) {
        const char* p = (k0 + 16 * ga + col == kn) ? knew_row + 16 * grp : kplane + gb[ga] + k_off;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) kr[ga][t] = *(const u32x4*)(p + 64 * t);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int key = k0 + 16 * (j >> 2) + 4 * grp + (j & 3);
        const char* p = key == kn ? vnew_row + 2 * (D / 16) * col
                                  : vplane + gb[j >> 2] + (int64_t)(j & 3) * row_bytes + v_off;
        vr[j] = *(const typename VRow<D>::T*)p;
    }
}

// An FP8 step's registers are widened to the bf16 operands of its MFMAs as they are used
// (every E4M3 value is a bf16 value, so the widening is exact): a K operand right before its
// S^T MFMA, a V word right before the byte permutes that take it, so no widened copy of the
// whole step is live at once.
template <int D, bool FP8>
__device__ __forceinline__ bf16x8 k_operand(const typename StepT<D, FP8>::K& x) {
    if constexpr (FP8)
        return __builtin_bit_cast(bf16x8, u32x4{e4m3x2_lo(x[0]), e4m3x2_hi(x[0]), e4m3x2_lo(x[1]), e4m3x2_hi(x[1])});
    else
        return __builtin_bit_cast(bf16x8, x);
}
// 32-bit word w (two bf16 dims) of a V row as the PV operand takes it
template <int D, bool FP8>
__device__ __forceinline__ uint32_t v_word(const typename StepT<D, FP8>::V& x, int w) {
    if constexpr (!FP8) {
        return x[w];
    } else if constexpr (D == 128) {
        return (w & 1) ? e4m3x2_hi(x[w >> 1]) : e4m3x2_lo(x[w >> 1]);
    } else {
        return (w & 1) ? e4m3x2_hi(x) : e4m3x2_lo(x);
    }
}

// Online-softmax update of one 32-key step (scores by MFMA, P packed to bf16, PV by MFMA).
// With ALiBi, sl2 = this lane's head slope in log2 units and pos the query's position: the
// score of key j gets sl2 * (j - pos) added after the scale.
template <int D, bool ALIBI, bool FP8>
__device__ __forceinline__ void compute_step(int k0, int kb, int ke, int grp, float c_log2, float sl2, int pos,
                                             const bf16x8 (&qf)[D / 32],
                                             typename StepT<D, FP8>::K (&kr)[2][D / 32],
                                             typename StepT<D, FP8>::V (&vr)[8],
                                             f32x4 (&oacc)[D / 16], float& m_run, float& l_run) {
    constexpr int KS = D / 32;
    constexpr int DPL = D / 16;
    typedef typename StepT<D, FP8>::V VT;
    const bool edge = (k0 < kb) || (k0 + 32 > ke);
    f32x4 sacc[2];
#pragma unroll
    for (int ga = 0; ga < 2; ++ga) {
        sacc[ga] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KS; ++t)
            sacc[ga] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<D, FP8>(kr[ga][t]), qf[t], sacc[ga], 0, 0, 0);
    }
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sc[j] = sacc[j >> 2][j & 3];
    if (edge) {
        // this lane's score j and V row j are the same key: k0 + 16*(j/4) + 4*grp + j%4
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = k0 + 16 * (j >> 2) + 4 * grp + (j & 3);
            const bool ok = key >= kb && key < ke;
            sc[j] = ok ? sc[j] : -INFINITY;
            vr[j] = ok ? vr[j] : (VT)(0u);
        }
    }
    float cs = c_log2;  // accumulator -> log2 units (1 once ALiBi has folded it in)
    if constexpr (ALIBI) {
        const float base = sl2 * (float)(k0 + 4 * grp - pos);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            sc[j] = fmaf(sc[j], c_log2, fmaf(sl2, (float)(16 * (j >> 2) + (j & 3)), base));
        cs = 1.f;
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mx = group4_max(mx);
    const float m_new = fmaxf(m_run, mx * cs);
    const float msub = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - msub);
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        pr[j] = __builtin_amdgcn_exp2f(fmaf(sc[j], cs, -msub));
        psum += pr[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
        for (int t = 0; t < DPL; ++t) oacc[t] *= alpha;
    }
    const u32x4 pw = {pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]), pack_bf16(pr[4], pr[5]),
                      pack_bf16(pr[6], pr[7])};
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
    for (int t = 0; t < DPL; ++t) {
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
        u32x4 w;
        w[0] = __builtin_amdgcn_perm(v_word<D, FP8>(vr[1], t >> 1), v_word<D, FP8>(vr[0], t >> 1), sel);
        w[1] = __builtin_amdgcn_perm(v_word<D, FP8>(vr[3], t >> 1), v_word<D, FP8>(vr[2], t >> 1), sel);
        w[2] = __builtin_amdgcn_perm(v_word<D, FP8>(vr[5], t >> 1), v_word<D, FP8>(vr[4], t >> 1), sel);
        w[3] = __builtin_amdgcn_perm(v_word<D, FP8>(vr[7], t >> 1), v_word<D, FP8>(vr[6], t >> 1), sel);
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), pb, oacc[t],
                                                          0, 0, 0);
    }
}

// ---------------------------------------------------------------- batch step list
// The 32-key steps of all sequences, in sequence order, form one list of S steps that is
// cut into nw equal chunks (chunk w = steps [w*S/nw, (w+1)*S/nw)), one per partition
// workgroup: every workgroup streams the same number of K/V rows whatever the length mix,
// and a chunk may end inside one sequence and start inside the next.  With nw no larger
// than the workgroups the device holds at once, all chunks run together and finish
// together.  A sequence cut by chunk boundaries leaves one partial state per chunk it
// touches: chunk w keeps its first sequence's in slot 0 and its last one's in slot 1.

__device__ inline int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    return v;
}

// Total steps S and chunks used, nw_eff = clamp(ceil(S / min_steps), 1, nw); also the steps
// of the sequences before `s_before` (pass num_seqs when not needed).  Wave-uniform.
__device__ inline void decode_chunking(const DecodeArgs& a, int lane, int s_before, int& S, int& nw,
                                       int& off) {
    int tot = 0, pre = 0;
    for (int c = 0; c < a.num_seqs; c += 64) {
        const int sl = c + lane;
        const int st = sl < a.num_seqs ? decode_steps(a.seq_lens[sl], a.window, a.key_start) : 0;
        tot += st;
        pre += sl < s_before ? st : 0;
    }
    S = __builtin_amdgcn_readfirstlane(wave_sum_i(tot));
    off = __builtin_amdgcn_readfirstlane(wave_sum_i(pre));
    const int want = (S + a.min_steps - 1) / a.min_steps;
    nw = max(1, min(a.nw, want));
}
__device__ inline int chunk_begin(int w, int S, int nw) { return (int)(((int64_t)w * S) / nw); }
// the chunk that holds step t, 0 <= t < S
__device__ inline int chunk_of(int t, int S, int nw) { return (int)(((int64_t)(t + 1) * nw - 1) / S); }

// Shared-prefix decode: fold the prefix chunks' states of query head `head` of sequence s
// into the running state (m_run, l_run, oacc) of this lane by log-sum-exp.  The sums go to
// the grp 0 lanes only: the partition kernel adds its per-lane partial sums over the four
// lane groups at the end.
template <int D>
__device__ __forceinline__ void fold_prefix(const DecodeArgs& a, int s, int head, int grp,
                                            f32x4 (&oacc)[D / 16], float& m_run, float& l_run) {
    constexpr int DPL = D / 16;
    const int64_t per_chunk = (int64_t)a.num_seqs * a.num_heads;
    const int64_t row = (int64_t)s * a.num_heads + head;
    float M = m_run;
    for (int c = 0; c < a.prefix_chunks; ++c) M = fmaxf(M, a.pre_ml[(c * per_chunk + row) * 2]);
    const float msub = M == -INFINITY ? 0.f : M;
    const float alpha = __builtin_amdgcn_exp2f(m_run - msub);
    float l = l_run * alpha;
#pragma unroll
    for (int t = 0; t < DPL; ++t) oacc[t] *= alpha;
    for (int c = 0; c < a.prefix_chunks; ++c) {
        const f32x2 ml = *(const f32x2*)(a.pre_ml + (c * per_chunk + row) * 2);
        const float w = __builtin_amdgcn_exp2f(ml[0] - msub);
        if (grp == 0) l = fmaf(w, ml[1], l);
        const float* po = a.pre_o + (c * per_chunk + row) * D;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d0 = DPL * (4 * grp + r);
#pragma unroll
            for (int t = 0; t < DPL; t += 4) {
                const f32x4 x = *(const f32x4*)(po + d0 + t);
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[t + i][r] = fmaf(w, x[i], oacc[t + i][r]);
            }
        }
    }
    m_run = M;
    l_run = l;
}

// 32-key steps per register set of an FP8 decode (1: as bf16; 2: the bytes of one bf16 step,
// measured slower)
constexpr int kDecodeFp8StepsPerSet = 1;

// CASCADE: shared-prefix decode.  Every sequence's steps then start at key_start, the first
// piece of a sequence folds the prefix's state into its own, and a sequence with no own key
// writes the prefix's result.
template <int D, bool ALIBI, bool CASCADE, bool FP8, bool FUSED>
__global__ __launch_bounds__(512) void decode_bf16_kernel(const DecodeArgs a) {
    static_assert(!FUSED || (!FP8 && !CASCADE), "the fused store serves the plain bf16 decode");
    constexpr int KS = D / 32;   // k-slices of q.K^T
    constexpr int DPL = D / 16;  // dims per lane chunk of a V row = PV MFMAs per step

    // one workgroup per (chunk of the step list, group of up to 8 KV heads); wave w serves
    // KV head 8*blockIdx.y + w, so the waves of a workgroup stream the same physical blocks
    // (all KV heads of a token row are adjacent) at the same time
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    // a wave past the last KV head runs the loop on the group's first head (its rows are
    // being read anyway) and writes nothing, so that every wave meets every barrier
    const bool wave_ok = blockIdx.y * 8 + (threadIdx.x >> 6) < a.c.num_kv_heads;
    const int g = wave_ok ? blockIdx.y * 8 + (threadIdx.x >> 6) : blockIdx.y * 8;
    int S, nw, unused;
    decode_chunking(a, lane, a.num_seqs, S, nw, unused);
    const int w = blockIdx.x;
    if (w >= nw) return;
    const int r0 = chunk_begin(w, S, nw);
    const int r1 = chunk_begin(w + 1, S, nw);
    const bool last_chunk = w == nw - 1;

    const int G = a.group;
    const int H = a.num_heads;
    const int head = g * G + col;
    const bool head_ok = wave_ok && col < G;
    const int BS = a.c.block_size;
    const int shift = a.c.block_shift;
    const int Hkv = a.c.num_kv_heads;
    const char* __restrict__ kplane = (const char*)a.c.kv;
    const char* __restrict__ vplane = kplane + a.c.plane_elems * (FP8 ? 1 : 2);
    // an FP8 cache holds K / kv_scale: the scale joins the softmax scale (and V's, the output's)
    const float c_log2 = a.scale * (FP8 ? a.c.kv_scale : 1.f) * 1.4426950408889634f;
    const float sl2 = ALIBI && head_ok ? a.alibi[head] * 1.4426950408889634f : 0.f;  // ALiBi slope, log2 units
    const int64_t row_elems = (int64_t)Hkv * D;
    const uint32_t row_bytes = (uint32_t)(row_elems * (FP8 ? 1 : 2));
    uint32_t k_off, v_off;
    lane_offsets<D, FP8>(col, grp, row_bytes, k_off, v_off);

    int carry = 0;  // steps of the sequences before chunk c of 64
    for (int c = 0; c < a.num_seqs; c += 64) {
        if (carry > r1 || (carry == r1 && !last_chunk)) break;
        const int sl = c + lane;
        const int n_l = sl < a.num_seqs ? a.seq_lens[sl] : 0;
        const int st_l = decode_steps(n_l, a.window, a.key_start);
        const int incl = wave_incl_scan(st_l, lane) + carry;
        const int off_l = incl - st_l;
        // sequences of this chunk: those whose steps meet [r0, r1); a sequence with no
        // steps (no keys) belongs to the chunk holding step off_l, or the last chunk
        const bool mine = sl < a.num_seqs &&
                          (st_l > 0 ? (off_l < r1 && incl > r0)
                                    : ((off_l >= r0 && off_l < r1) || (last_chunk && off_l == S)));
        uint64_t mask = __ballot(mine);
        carry = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
        while (mask) {
            const int l = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)mask) - 1);
            mask &= mask - 1;
            const int s = c + l;
            const int n = __builtin_amdgcn_readlane(n_l, l);
            const int steps = __builtin_amdgcn_readlane(st_l, l);
            const int off = __builtin_amdgcn_readlane(off_l, l);
            __bf16* out_row = (__bf16*)a.out + ((int64_t)s * H + head) * D;
            if (steps == 0) {  // no key of its own: the prefix's result, or a zero row
                if constexpr (CASCADE) {
                    f32x4 oacc[DPL];
#pragma unroll
                    for (int t = 0; t < DPL; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                    float m_run = -INFINITY, l_run = 0.f;
                    fold_prefix<D>(a, s, head_ok ? head : g * G, grp, oacc, m_run, l_run);
                    const float l_tot = group4_sum(l_run);
                    const float inv = l_tot > 0.f ? (FP8 ? a.c.kv_scale : 1.f) / l_tot : 0.f;
                    if (head_ok) {
                        for (int r = 0; r < 4; ++r) {
                            const int d0 = DPL * (4 * grp + r);
                            for (int t = 0; t < DPL; ++t) out_row[d0 + t] = (__bf16)(oacc[t][r] * inv);
                        }
                    }
                } else if (head_ok) {
                    for (int r = 0; r < 4; ++r) {
                        const int d0 = DPL * (4 * grp + r);
                        for (int t = 0; t < DPL; ++t) out_row[d0 + t] = (__bf16)0.f;
                    }
                }
                continue;
            }
            const int ls = max(r0 - off, 0);
            const int le = min(r1 - off, steps);
            const int lo = decode_lo(n, a.window, a.key_start);
            const int base = decode_base(lo);
            const int step_begin = base + 32 * ls;             // multiple of 32
            const int kb = step_begin > lo ? step_begin : lo;  // first live key of the segment
            const int ke = min(n, base + 32 * le);             // one past the last
            const const_table_t table = (const_table_t)(a.table + (int64_t)s * a.max_blocks);
            // fused store: this workgroup holds the sequence's last step (the new token's key)
            const bool new_here = FUSED && le == steps;
            const int k_last = base + 32 * (steps - 1);
            const char* knew_row = FUSED ? (const char*)a.knew + ((int64_t)s * Hkv + g) * D * 2 : nullptr;
            const char* vnew_row = FUSED ? (const char*)a.vnew + ((int64_t)s * Hkv + g) * D * 2 : nullptr;

            // Q^T operand: head col, the dims of k-slice t (q_slice)
            bf16x8 qf[KS];
            {
                const u32x4* qrow = (const u32x4*)((const __bf16*)a.q + ((int64_t)s * H + (head_ok ? head : g * G)) * D);
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    const u32x4 x = qrow[q_slice<FP8>(t, grp)];
                    qf[t] = __builtin_bit_cast(bf16x8, head_ok ? x : (u32x4)(0u));
                }
            }

            f32x4 oacc[DPL];
#pragma unroll
            for (int t = 0; t < DPL; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            float m_run = -INFINITY;
            float l_run = 0.f;

            // Two register sets: the loads of step i+1 are in flight while step i computes.
            // The prefetch is unconditional so that every iteration issues the same number of
            // loads and the waits stay exact: after the last step it is a dummy in which every
            // lane reads the same few 16-byte pieces of rows the step already read (a re-read
            // of the step's whole rows missed the L2 often enough to add ~4% to the traffic).  A
            // workgroup barrier per two steps keeps the 8 waves, which read adjacent 256-byte
            // pieces of the same 2 KB token rows, close together in the key walk (measured: 3%
            // more bandwidth than free-running waves).
            // A register set holds SPS consecutive steps (an FP8 set may hold two, the bytes of one
            // bf16 step); a step of a set past the segment's end is loaded as a dummy and not
            // computed.
            constexpr int SPS = FP8 ? kDecodeFp8StepsPerSet : 1;
            constexpr int SK = 32 * SPS;
            typename StepT<D, FP8>::K kA[SPS][2][KS], kB[SPS][2][KS];
            typename StepT<D, FP8>::V vA[SPS][8], vB[SPS][8];
            int k0 = step_begin;
            auto ld = [&](int k, auto& kr, auto& vr, bool dummy) {
                if constexpr (FUSED) {
                    if (!dummy && new_here && k == k_last) {
                        load_step_new<D>(k, kb, ke, table, shift, BS, row_elems, g, kplane, vplane, k_off, v_off,
                                         row_bytes, col, grp, n - 1, knew_row, vnew_row, kr, vr);
                        return;
                    }
                }
                load_step<D, FP8>(k, kb, ke, table, shift, BS, row_elems, g, kplane, vplane, dummy ? 0u : k_off,
                                  dummy ? 0u : v_off, row_bytes, kr, vr);
            };
            // the SPS steps of the set at k (k < ke), or dummies at k
            auto ld_set = [&](int k, auto& kr, auto& vr, bool dummy) {
#pragma unroll
                for (int u = 0; u < SPS; ++u) {
                    const bool past = dummy || k + 32 * u >= ke;
                    ld(past ? k : k + 32 * u, kr[u], vr[u], past);
                }
            };
            auto compute_set = [&](int k, auto& kr, auto& vr) {
#pragma unroll
                for (int u = 0; u < SPS; ++u)
                    if (u == 0 || k + 32 * u < ke)
                        compute_step<D, ALIBI, FP8>(k + 32 * u, kb, ke, grp, c_log2, sl2, n - 1, qf, kr[u], vr[u], oacc,
                                                    m_run, l_run);
            };
            ld_set(k0, kA, vA, false);
            while (true) {
                __syncthreads();
                const bool more1 = k0 + SK < ke;
                ld_set(more1 ? k0 + SK : k0, kB, vB, !more1);
                compute_set(k0, kA, vA);
                k0 += SK;
                if (k0 >= ke) break;
                const bool more2 = k0 + SK < ke;
                ld_set(more2 ? k0 + SK : k0, kA, vA, !more2);
                compute_set(k0, kB, vB);
                k0 += SK;
                if (k0 >= ke) break;
            }

            if constexpr (FUSED) {  // the new token's rows into its cache slot (KV head g's part)
                if (new_here && wave_ok && lane < D / 8) {
                    const int slot = a.slots[s];
                    if (slot >= 0) {
                        const int64_t dst = ((int64_t)slot * Hkv + g) * D * 2 + 16 * lane;
                        *(u32x4*)((char*)a.c.kv + dst) = *(const u32x4*)(knew_row + 16 * lane);
                        *(u32x4*)((char*)a.c.kv + a.c.plane_elems * 2 + dst) = *(const u32x4*)(vnew_row + 16 * lane);
                    }
                }
            }
            if constexpr (CASCADE) {  // the sequence's first piece also holds the prefix
                if (ls == 0) fold_prefix<D>(a, s, head_ok ? head : g * G, grp, oacc, m_run, l_run);
            }
            const float l_tot = group4_sum(l_run);
            if (head_ok) {
                if (ls == 0 && le == steps) {  // the whole sequence: normalised output
                    const float inv = l_tot > 0.f ? (FP8 ? a.c.kv_scale : 1.f) / l_tot : 0.f;
                    for (int r = 0; r < 4; ++r) {
                        const int d0 = DPL * (4 * grp + r);
                        uint32_t wv[DPL / 2];
                        for (int t = 0; t < DPL / 2; ++t)
                            wv[t] = pack_bf16(oacc[2 * t][r] * inv, oacc[2 * t + 1][r] * inv);
                        if constexpr (DPL == 8)
                            *(u32x4*)(out_row + d0) = u32x4{wv[0], wv[1], wv[2], wv[3]};
                        else
                            *(u32x2*)(out_row + d0) = u32x2{wv[0], wv[1]};
                    }
                } else {  // a piece: partial state into this chunk's slot
                    const int64_t slot = ((int64_t)(2 * w + (off <= r0 ? 0 : 1))) * H + head;
                    float* wo = a.ws_o + slot * D;
                    for (int r = 0; r < 4; ++r) {
                        const int d0 = DPL * (4 * grp + r);
                        for (int t = 0; t < DPL; t += 4)
                            *(f32x4*)(wo + d0 + t) = f32x4{oacc[t][r], oacc[t + 1][r], oacc[t + 2][r], oacc[t + 3][r]};
                    }
                    if (grp == 0) *(f32x2*)(a.ws_ml + slot * 2) = f32x2{m_run, l_tot};
                }
            }
        }
    }
}

// Shared-prefix pass.  The rows of KV head g are its (sequence, query head) pairs,
// r = s*G + (head - g*G); a wave takes 16 of them as the 16 MFMA columns that the partition
// kernel gives to the query heads of one group, so each K/V row it loads serves 16 queries
// (the prefix is the same keys for every sequence: this is a dense contraction).
// Workgroup = (KV head g, prefix chunk c, row group rg): its 8 waves split the chunk's 32-key
// steps, then combine their states by log-sum-exp through LDS in three halving rounds, and
// wave 0 writes the chunk's state.  Workgroup ids are dealt to the 8 XCDs in turn; they are
// mapped so that all row groups of one (g, c) run on the same XCD, where the chunk's K/V is
// read from HBM once and from that XCD's L2 by the other row groups.
template <int D, bool FP8>
__global__ __launch_bounds__(512) void cascade_prefix_kernel(const DecodeArgs a, int row_groups) {
    constexpr int KS = D / 32;
    constexpr int DPL = D / 16;
    __shared__ float red[4][4 * DPL + 2][64];
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int wave = threadIdx.x >> 6;
    const int Hkv = a.c.num_kv_heads;
    const int k = blockIdx.x >> 3;
    const int u = (blockIdx.x & 7) + 8 * (k / row_groups);
    const int rg = k % row_groups;
    if (u >= Hkv * a.prefix_chunks) return;  // whole workgroup, before any barrier
    const int g = u % Hkv;
    const int c = u / Hkv;
    const int G = a.group;
    const int H = a.num_heads;
    const int row = 16 * rg + col;
    const bool row_ok = row < a.num_seqs * G;
    const int s = row_ok ? row / G : 0;
    const int head = g * G + (row_ok ? row % G : 0);
    const int P = a.key_start;
    const int Ps = (P + 31) >> 5;
    const int cb = (int)((int64_t)c * Ps / a.prefix_chunks);
    const int ce = (int)((int64_t)(c + 1) * Ps / a.prefix_chunks);
    const int st0 = cb + (ce - cb) * wave / 8;
    const int st1 = cb + (ce - cb) * (wave + 1) / 8;
    const int kb = 32 * st0;
    const int ke = min(P, 32 * st1);

    const int BS = a.c.block_size;
    const int shift = a.c.block_shift;
    const char* __restrict__ kplane = (const char*)a.c.kv;
    const char* __restrict__ vplane = kplane + a.c.plane_elems * (FP8 ? 1 : 2);
    // an FP8 cache holds K / kv_scale: the scale joins the softmax scale (and V's, the output's)
    const float c_log2 = a.scale * (FP8 ? a.c.kv_scale : 1.f) * 1.4426950408889634f;
    const int64_t row_elems = (int64_t)Hkv * D;
    const uint32_t row_bytes = (uint32_t)(row_elems * (FP8 ? 1 : 2));
    uint32_t k_off, v_off;
    lane_offsets<D, FP8>(col, grp, row_bytes, k_off, v_off);

    bf16x8 qf[KS];
    {
        const u32x4* qrow = (const u32x4*)((const __bf16*)a.q + ((int64_t)s * H + head) * D);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const u32x4 x = qrow[q_slice<FP8>(t, grp)];
            qf[t] = __builtin_bit_cast(bf16x8, row_ok ? x : (u32x4)(0u));
        }
    }
    f32x4 oacc[DPL];
#pragma unroll
    for (int t = 0; t < DPL; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;
    if (st1 > st0) {
        // the waves read different keys, so they run free (no barrier in the walk)
        typename StepT<D, FP8>::K kA[2][KS], kB[2][KS];
            typename StepT<D, FP8>::V vA[8], vB[8];
        int k0 = kb;
        load_step<D, FP8>(k0, kb, ke, (const_table_t)a.table, shift, BS, row_elems, g, kplane, vplane, k_off, v_off, row_bytes, kA, vA);
        while (true) {
            const int n1 = k0 + 32 < ke ? k0 + 32 : k0;
            load_step<D, FP8>(n1, kb, ke, (const_table_t)a.table, shift, BS, row_elems, g, kplane, vplane, k_off, v_off, row_bytes, kB, vB);
            compute_step<D, false, FP8>(k0, kb, ke, grp, c_log2, 0.f, 0, qf, kA, vA, oacc, m_run, l_run);
            k0 += 32;
            if (k0 >= ke) break;
            const int n2 = k0 + 32 < ke ? k0 + 32 : k0;
            load_step<D, FP8>(n2, kb, ke, (const_table_t)a.table, shift, BS, row_elems, g, kplane, vplane, k_off, v_off, row_bytes, kA, vA);
            compute_step<D, false, FP8>(k0, kb, ke, grp, c_log2, 0.f, 0, qf, kB, vB, oacc, m_run, l_run);
            k0 += 32;
            if (k0 >= ke) break;
        }
    }
    // waves [half, 2*half) hand their states to waves [0, half)
#pragma unroll
    for (int half = 4; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) {
            float (*slot)[64] = red[wave - half];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < DPL; ++t) slot[r * DPL + t][lane] = oacc[t][r];
            slot[4 * DPL][lane] = m_run;
            slot[4 * DPL + 1][lane] = l_run;
        }
        __syncthreads();
        if (wave < half) {
            float (*slot)[64] = red[wave];
            const float mo = slot[4 * DPL][lane];
            const float M = fmaxf(m_run, mo);
            const float msub = M == -INFINITY ? 0.f : M;
            const float a0 = __builtin_amdgcn_exp2f(m_run - msub);
            const float a1 = __builtin_amdgcn_exp2f(mo - msub);
            l_run = fmaf(l_run, a0, slot[4 * DPL + 1][lane] * a1);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < DPL; ++t) oacc[t][r] = fmaf(oacc[t][r], a0, slot[r * DPL + t][lane] * a1);
            m_run = M;
        }
        __syncthreads();
    }
    if (wave != 0) return;
    const float l_tot = group4_sum(l_run);
    if (!row_ok) return;
    const int64_t st = ((int64_t)c * a.num_seqs + s) * H + head;
    float* po = a.pre_o + st * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int d0 = DPL * (4 * grp + r);
#pragma unroll
        for (int t = 0; t < DPL; t += 4)
            *(f32x4*)(po + d0 + t) = f32x4{oacc[t][r], oacc[t + 1][r], oacc[t + 2][r], oacc[t + 3][r]};
    }
    if (grp == 0) *(f32x2*)(a.pre_ml + st * 2) = f32x2{m_run, l_tot};
}

// Merge of the pieces of a sequence cut by chunk boundaries (log-sum-exp rescale by
// exp2(m_p - max m)): a workgroup of MW waves per (sequence, four query heads); in each wave
// lanes 16h .. 16h+15 take query head 4*blockIdx.y + h, D/16 dims each.  Wave w folds pieces
// w, w + MW, ... loading MP of them per memory round trip, with a running maximum; the MW
// partial states are then combined through LDS by wave 0.  MW = 4 when sequences are cut
// into many pieces (few long sequences), else 1.
template <int D, int MW>
__global__ __launch_bounds__(64 * MW) void decode_merge_kernel(const DecodeArgs a) {
    constexpr int DL = D / 16;
    constexpr int MP = 8;  // pieces loaded per memory round trip
    __shared__ float red[MW > 1 ? MW : 1][2 + DL][64];
    const int s = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wv_id = threadIdx.x >> 6;
    int S, nw, off;
    decode_chunking(a, lane, s, S, nw, off);
    const int steps = decode_steps(a.seq_lens[s], a.window, a.key_start);
    if (steps == 0) return;
    const int w_lo = chunk_of(off, S, nw);
    const int np = chunk_of(off + steps - 1, S, nw) - w_lo + 1;
    if (np <= 1) return;  // written whole by its chunk
    const int h_lane = blockIdx.y * 4 + (lane >> 4);
    const bool h_ok = h_lane < a.num_heads;
    const int h = h_ok ? h_lane : a.num_heads - 1;
    // piece q lives in chunk w_lo + q, slot 0, except the first when the sequence starts
    // after that chunk's first step (then it is that chunk's last sequence: slot 1)
    const int first_slot = off > chunk_begin(w_lo, S, nw) ? 1 : 0;
    const int d0 = (lane & 15) * DL;
    float M = -INFINITY, L = 0.f;
    float acc[DL];
#pragma unroll
    for (int t = 0; t < DL; ++t) acc[t] = 0.f;
    const int nmine = np > wv_id ? (np - wv_id + MW - 1) / MW : 0;  // pieces of this wave
    for (int k0 = 0; k0 < nmine; k0 += MP) {
        f32x2 mv[MP];
        f32x4 ov[MP][DL / 4];
#pragma unroll
        for (int j = 0; j < MP; ++j) {
            const int q = wv_id + MW * min(k0 + j, nmine - 1);
            const int64_t slot = ((int64_t)(2 * (w_lo + q) + (q == 0 ? first_slot : 0))) * a.num_heads + h;
            mv[j] = *(const f32x2*)(a.ws_ml + slot * 2);
#pragma unroll
            for (int t = 0; t < DL / 4; ++t) ov[j][t] = *(const f32x4*)(a.ws_o + slot * D + d0 + 4 * t);
        }
        float mj[MP];
        float Mn = M;
#pragma unroll
        for (int j = 0; j < MP; ++j) {
            mj[j] = k0 + j < nmine ? mv[j][0] : -INFINITY;
            Mn = fmaxf(Mn, mj[j]);
        }
        const float msub = Mn == -INFINITY ? 0.f : Mn;
        const float alpha = __builtin_amdgcn_exp2f(M - msub);
        L *= alpha;
#pragma unroll
        for (int t = 0; t < DL; ++t) acc[t] *= alpha;
#pragma unroll
        for (int j = 0; j < MP; ++j) {
            const float wq = __builtin_amdgcn_exp2f(mj[j] - msub);
            L = fmaf(wq, mv[j][1], L);
#pragma unroll
            for (int t = 0; t < DL; ++t) acc[t] = fmaf(wq, ov[j][t / 4][t % 4], acc[t]);
        }
        M = Mn;
    }
    float Lt = L;
    if constexpr (MW > 1) {
        red[wv_id][0][lane] = M;
        red[wv_id][1][lane] = L;
#pragma unroll
        for (int t = 0; t < DL; ++t) red[wv_id][2 + t][lane] = acc[t];
        __syncthreads();
        if (wv_id != 0) return;
        float Mt = red[0][0][lane];
#pragma unroll
        for (int w = 1; w < MW; ++w) Mt = fmaxf(Mt, red[w][0][lane]);
        Lt = 0.f;
#pragma unroll
        for (int t = 0; t < DL; ++t) acc[t] = 0.f;
#pragma unroll
        for (int w = 0; w < MW; ++w) {
            const float sc = __builtin_amdgcn_exp2f(red[w][0][lane] - Mt);  // 0 for a wave with no piece
            Lt = fmaf(sc, red[w][1][lane], Lt);
#pragma unroll
            for (int t = 0; t < DL; ++t) acc[t] = fmaf(sc, red[w][2 + t][lane], acc[t]);
        }
    }
    if (!h_ok) return;
    const float inv = Lt > 0.f ? a.c.kv_scale / Lt : 0.f;  // an FP8 cache holds V / kv_scale
    uint32_t wv[DL / 2];
#pragma unroll
    for (int t = 0; t < DL / 2; ++t) wv[t] = pack_bf16(acc[2 * t] * inv, acc[2 * t + 1] * inv);
    __bf16* out = (__bf16*)a.out + ((int64_t)s * a.num_heads + h) * D + d0;
    if constexpr (DL == 8)
        *(u32x4*)out = u32x4{wv[0], wv[1], wv[2], wv[3]};
    else
        *(u32x2*)out = u32x2{wv[0], wv[1]};
}

int decode_resident_slots(int head_size, int num_kv_heads) {
    // per device and (head size, waves per workgroup): compute units x resident workgroups per
    // unit, 0 = not yet queried.  Relaxed atomics: concurrent first calls from several host
    // threads may each query, and all store the same value.
    static std::atomic<int> slots[64][2][9];
    const int waves = num_kv_heads < 8 ? num_kv_heads : 8;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || waves < 1) {
        (void)hipGetLastError();
        return 256;
    }
    const int di = head_size == 128 ? 1 : 0;
    int v = slots[dev][di][waves].load(std::memory_order_relaxed);
    if (v == 0) {
        int ncu = 0, nb = 0;
        hipError_t e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = head_size == 128
                    ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_bf16_kernel<128, false, false, false, false>, 64 * waves, 0)
                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_bf16_kernel<64, false, false, false, false>, 64 * waves, 0);
        if (e != hipSuccess || ncu <= 0 || nb <= 0) {
            (void)hipGetLastError();
            return 256;
        }
        v = ncu * nb;
        slots[dev][di][waves].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Partition kernel (+ merge kernel when the batch is cut into more than one chunk).
template <bool ALIBI, bool CASCADE, bool FP8, bool FUSED = false>
static void launch_partition_merge(const DecodeArgs& a, hipStream_t st) {
    const int hkv = a.c.num_kv_heads;
    const dim3 grid(a.nw, (hkv + 7) / 8);
    const dim3 block(64 * (hkv < 8 ? hkv : 8));
    if (a.c.head_size == 128)
        hipLaunchKernelGGL((decode_bf16_kernel<128, ALIBI, CASCADE, FP8, FUSED>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((decode_bf16_kernel<64, ALIBI, CASCADE, FP8, FUSED>), grid, block, 0, st, a);
    if (a.nw > 1) {
        const dim3 mg(a.num_seqs, (a.num_heads + 3) / 4);
        const bool many = a.nw > 8 * a.num_seqs;  // more than ~8 pieces per sequence
        if (a.c.head_size == 128) {
            if (many) hipLaunchKernelGGL((decode_merge_kernel<128, 4>), mg, dim3(256), 0, st, a);
            else hipLaunchKernelGGL((decode_merge_kernel<128, 1>), mg, dim3(64), 0, st, a);
        } else {
            if (many) hipLaunchKernelGGL((decode_merge_kernel<64, 4>), mg, dim3(256), 0, st, a);
            else hipLaunchKernelGGL((decode_merge_kernel<64, 1>), mg, dim3(64), 0, st, a);
        }
    }
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t st) {
    const bool fp8 = a.c.dtype == 2;
    if (a.knew != nullptr && !fp8) {  // the store fused into the partition kernel
        if (a.alibi) launch_partition_merge<true, false, false, true>(a, st);
        else launch_partition_merge<false, false, false, true>(a, st);
        return hipGetLastError();
    }
    if (a.alibi) {
        if (fp8) launch_partition_merge<true, false, true>(a, st);
        else launch_partition_merge<true, false, false>(a, st);
    } else {
        if (fp8) launch_partition_merge<false, false, true>(a, st);
        else launch_partition_merge<false, false, false>(a, st);
    }
    return hipGetLastError();
}

hipError_t launch_prefix_pass(const DecodeArgs& a, hipStream_t st) {
    const bool fp8 = a.c.dtype == 2;
    if (a.prefix_mfma) return launch_prefix_states(a, st);
    {
        const int row_groups = (a.num_seqs * a.group + 15) / 16;
        const int units = a.c.num_kv_heads * a.prefix_chunks;
        const dim3 grid((unsigned)(8LL * row_groups * ((units + 7) / 8)));
        if (a.c.head_size == 128) {
            if (fp8) hipLaunchKernelGGL((cascade_prefix_kernel<128, true>), grid, dim3(512), 0, st, a, row_groups);
            else hipLaunchKernelGGL((cascade_prefix_kernel<128, false>), grid, dim3(512), 0, st, a, row_groups);
        } else {
            if (fp8) hipLaunchKernelGGL((cascade_prefix_kernel<64, true>), grid, dim3(512), 0, st, a, row_groups);
            else hipLaunchKernelGGL((cascade_prefix_kernel<64, false>), grid, dim3(512), 0, st, a, row_groups);
        }
    }
    return hipGetLastError();
}

hipError_t launch_cascade_decode_bf16(const DecodeArgs& a, hipStream_t st) {
    const bool fp8 = a.c.dtype == 2;
    const hipError_t e = launch_prefix_pass(a, st);
    if (e != hipSuccess) return e;
    if (fp8) launch_partition_merge<false, true, true>(a, st);
    else launch_partition_merge<false, true, false>(a, st);
    return hipGetLastError();
}

}  // namespace pa
