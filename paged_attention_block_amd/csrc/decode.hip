// Grouped-query paged decode for bf16 caches on gfx950: split-K partitions + log-sum-exp merge.
//
// The operation (MinivLLM API docs, "Attention", paged_attention_decode): one query per
// sequence, attending its seq_lens[s] cached keys through the block table, online softmax.
// Long contexts are split over the key axis (vLLM learning book section 7: split-KV wins
// small-batch long-sequence decode); each partition leaves (m, l, O) and a merge rescales
// them by exp2(m_p - max m).
//
// Work item = one wavefront per (sequence s, KV head g, partition p).  All G query heads of
// the group share every K/V row the wave streams, so each KV byte is read from HBM once.
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

#include "pa_internal.hpp"

namespace pa {

namespace {

__device__ inline float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ inline float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ inline uint32_t pack_bf16(float lo, float hi) { return pack_bf16x2(lo, hi); }

// DPL = dims per lane chunk of a V row: 8 (16 B) for D = 128, 4 (8 B) for D = 64.
template <int D> struct VRow;
template <> struct VRow<128> { typedef u32x4 T; };
template <> struct VRow<64> { typedef u32x2 T; };

}  // namespace

// Loads of the 32-key step at k0 into registers: K rows (2 groups of 16 keys x KS slices,
// MFMA A-operand layout) and the V rows one lane needs for the PV MFMAs (8 keys x DPL
// dims).  Both 16-key groups of a step lie in one physical block each (block_size >= 16,
// 16-aligned); a group with no live key is never looked up and its lanes read the other
// group's rows instead, so every load is in bounds and unconditional.  Keys outside
// [kb, ke) are masked after the load.
template <int D>
__device__ __forceinline__ void load_step(int k0, int kb, int ke, const int32_t* __restrict__ table,
                                          int shift, int BS, int64_t row_elems, int g,
                                          const char* __restrict__ kplane,
                                          const char* __restrict__ vplane, uint32_t k_off,
                                          uint32_t v_off, uint32_t row_bytes,
                                          u32x4 (&kr)[2][D / 32], typename VRow<D>::T (&vr)[8]) {
    typedef typename VRow<D>::T VT;
    // wave-uniform byte offset of (first key of each 16-key group, KV head g) in a plane
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
        const char* base = kplane + gb[ga];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) kr[ga][t] = *(const u32x4*)(base + k_off + 64 * t);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const char* base = vplane + gb[j >> 2] + (int64_t)(j & 3) * row_bytes;
        vr[j] = *(const VT*)(base + v_off);
    }
}

// Online-softmax update of one 32-key step (scores by MFMA, P packed to bf16, PV by MFMA).
template <int D>
__device__ __forceinline__ void compute_step(int k0, int kb, int ke, int grp, float c_log2,
                                             const bf16x8 (&qf)[D / 32], u32x4 (&kr)[2][D / 32],
                                             typename VRow<D>::T (&vr)[8], f32x4 (&oacc)[D / 16],
                                             float& m_run, float& l_run) {
    constexpr int KS = D / 32;
    constexpr int DPL = D / 16;
    typedef typename VRow<D>::T VT;
    const bool edge = (k0 < kb) || (k0 + 32 > ke);
    f32x4 sacc[2];
#pragma unroll
    for (int ga = 0; ga < 2; ++ga) {
        sacc[ga] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KS; ++t)
            sacc[ga] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[ga][t]),
                                                               qf[t], sacc[ga], 0, 0, 0);
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
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c_log2);
    const float msub = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - msub);
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        pr[j] = __builtin_amdgcn_exp2f(fmaf(sc[j], c_log2, -msub));
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
        w[0] = __builtin_amdgcn_perm(vr[1][t >> 1], vr[0][t >> 1], sel);
        w[1] = __builtin_amdgcn_perm(vr[3][t >> 1], vr[2][t >> 1], sel);
        w[2] = __builtin_amdgcn_perm(vr[5][t >> 1], vr[4][t >> 1], sel);
        w[3] = __builtin_amdgcn_perm(vr[7][t >> 1], vr[6][t >> 1], sel);
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), pb, oacc[t],
                                                          0, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(512) void decode_bf16_kernel(const DecodeArgs a) {
    constexpr int KS = D / 32;   // k-slices of q.K^T
    constexpr int DPL = D / 16;  // dims per lane chunk of a V row = PV MFMAs per step
    typedef typename VRow<D>::T VT;

    // one workgroup per (sequence, group of up to 8 KV heads, partition); wave w serves KV
    // head 8*blockIdx.y + w, so the waves of a workgroup stream the same physical blocks
    // (all KV heads of a token row are adjacent) at the same time
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int s = blockIdx.x;
    const int g = blockIdx.y * 8 + (threadIdx.x >> 6);
    const int p = blockIdx.z;
    if (g >= a.c.num_kv_heads) return;

    const int n = a.seq_lens[s];
    const int G = a.group;
    const int H = a.num_heads;
    const int head = g * G + col;
    const bool head_ok = col < G;
    __bf16* out_row = (__bf16*)a.out + ((int64_t)s * H + head) * D;

    if (n <= 0) {  // zero-length sequence: zero output row
        if (p == 0 && head_ok) {
            for (int r = 0; r < 4; ++r) {
                const int d0 = DPL * (4 * grp + r);
                for (int t = 0; t < DPL; ++t) out_row[d0 + t] = (__bf16)0.f;
            }
        }
        return;
    }
    const int lo = decode_lo(n, a.window);
    const int base = decode_base(lo);
    const int nparts = (n - base + a.part - 1) / a.part;
    if (p >= nparts || p >= a.max_parts) return;
    const int step_begin = base + p * a.part;            // multiple of 32
    const int kb = step_begin > lo ? step_begin : lo;    // first live key of the partition
    const int ke = min(n, step_begin + a.part);          // one past the last

    const int BS = a.c.block_size;
    const int shift = a.c.block_shift;
    const int Hkv = a.c.num_kv_heads;
    const char* __restrict__ kplane = (const char*)a.c.kv;
    const char* __restrict__ vplane = kplane + a.c.plane_elems * 2;
    const int32_t* __restrict__ table = a.table + (int64_t)s * a.max_blocks;
    const float c_log2 = a.scale * 1.4426950408889634f;
    // per-lane byte offsets from a group's first row: K rows (key col, dims 8*grp of each
    // 32-dim slice), V rows (key 4*grp + j%4, dims DPL*col)
    const int64_t row_elems = (int64_t)Hkv * D;
    const uint32_t row_bytes = (uint32_t)(row_elems * 2);
    const uint32_t k_off = (uint32_t)col * row_bytes + 16u * grp;
    const uint32_t v_off = (uint32_t)(4 * grp) * row_bytes + 2u * DPL * col;

    // Q^T operand: head col, dims 32t + 8*grp .. +8
    bf16x8 qf[KS];
    {
        const u32x4* qrow = (const u32x4*)((const __bf16*)a.q + ((int64_t)s * H + (head_ok ? head : g * G)) * D);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const u32x4 x = qrow[4 * t + grp];
            qf[t] = __builtin_bit_cast(bf16x8, head_ok ? x : (u32x4)(0u));
        }
    }

    f32x4 oacc[DPL];
#pragma unroll
    for (int t = 0; t < DPL; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // Two register sets: the loads of step i+1 are in flight while step i computes.  The
    // prefetch is unconditional (the last step re-reads its own rows, which hit in cache)
    // so that every iteration issues the same number of loads and the waits stay exact.
    u32x4 kA[2][KS], kB[2][KS];
    VT vA[8], vB[8];
    int k0 = step_begin;
    load_step<D>(k0, kb, ke, table, shift, BS, row_elems, g, kplane, vplane, k_off, v_off, row_bytes, kA, vA);
    while (true) {
        const int n1 = k0 + 32 < ke ? k0 + 32 : k0;
        load_step<D>(n1, kb, ke, table, shift, BS, row_elems, g, kplane, vplane, k_off, v_off, row_bytes, kB, vB);
        compute_step<D>(k0, kb, ke, grp, c_log2, qf, kA, vA, oacc, m_run, l_run);
        k0 += 32;
        if (k0 >= ke) break;
        const int n2 = k0 + 32 < ke ? k0 + 32 : k0;
        load_step<D>(n2, kb, ke, table, shift, BS, row_elems, g, kplane, vplane, k_off, v_off, row_bytes, kA, vA);
        compute_step<D>(k0, kb, ke, grp, c_log2, qf, kB, vB, oacc, m_run, l_run);
        k0 += 32;
        if (k0 >= ke) break;
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!head_ok) return;

    if (nparts == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        for (int r = 0; r < 4; ++r) {
            const int d0 = DPL * (4 * grp + r);
            uint32_t w[DPL / 2];
            for (int t = 0; t < DPL / 2; ++t)
                w[t] = pack_bf16(oacc[2 * t][r] * inv, oacc[2 * t + 1][r] * inv);
            if constexpr (DPL == 8)
                *(uint4*)(out_row + d0) = make_uint4(w[0], w[1], w[2], w[3]);
            else
                *(uint2*)(out_row + d0) = make_uint2(w[0], w[1]);
        }
    } else {
        const int64_t slot = ((int64_t)s * H + head) * a.max_parts + p;
        float* wo = a.ws_o + slot * D;
        for (int r = 0; r < 4; ++r) {
            const int d0 = DPL * (4 * grp + r);
            for (int t = 0; t < DPL; t += 4)
                *(float4*)(wo + d0 + t) =
                    make_float4(oacc[t][r], oacc[t + 1][r], oacc[t + 2][r], oacc[t + 3][r]);
        }
        if (grp == 0) *(float2*)(a.ws_ml + slot * 2) = make_float2(m_run, l_tot);
    }
}

// Merge of the partition states of one (sequence, head): one wavefront, D/64 dims per lane.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const DecodeArgs a) {
    const int s = blockIdx.x;
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int np = min(decode_num_parts(a.seq_lens[s], a.window, a.part), a.max_parts);
    if (np <= 1) return;
    const int64_t slot0 = ((int64_t)s * a.num_heads + h) * a.max_parts;
    const float2* ml = (const float2*)(a.ws_ml + slot0 * 2);
    float M = -INFINITY;
    for (int p = lane; p < np; p += 64) M = fmaxf(M, ml[p].x);
    M = wave_max(M);
    float L = 0.f;
    for (int p = lane; p < np; p += 64) L += ml[p].y * __builtin_amdgcn_exp2f(ml[p].x - M);
    L = wave_sum(L);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float* wo = a.ws_o + slot0 * D;
    __bf16* out = (__bf16*)a.out + ((int64_t)s * a.num_heads + h) * D;
    for (int d = lane; d < D; d += 64) {
        float acc = 0.f;
        for (int p = 0; p < np; ++p) acc += wo[(int64_t)p * D + d] * __builtin_amdgcn_exp2f(ml[p].x - M);
        out[d] = (__bf16)(acc * inv);
    }
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t st) {
    const int hkv = a.c.num_kv_heads;
    const dim3 grid(a.num_seqs, (hkv + 7) / 8, a.max_parts);
    const dim3 block(64 * (hkv < 8 ? hkv : 8));
    if (a.c.head_size == 128)
        hipLaunchKernelGGL(decode_bf16_kernel<128>, grid, block, 0, st, a);
    else
        hipLaunchKernelGGL(decode_bf16_kernel<64>, grid, block, 0, st, a);
    if (a.max_parts > 1) {
        const dim3 mg(a.num_seqs, a.num_heads);
        if (a.c.head_size == 128)
            hipLaunchKernelGGL(decode_merge_kernel<128>, mg, dim3(64), 0, st, a);
        else
            hipLaunchKernelGGL(decode_merge_kernel<64>, mg, dim3(64), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace pa
