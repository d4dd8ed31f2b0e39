// Varlen causal paged prefill for bf16 caches on gfx950 (MFMA, fp32 online softmax).
//
// The operation (MinivLLM API docs, "Attention", flash_attention_prefill; HF transformers
// continuous_batching input_ouputs.py, build_attention_mask): packed query chunks, causal
// diagonal offset by seqlen_k - seqlen_q, optional sliding window of W keys ending at the
// query's own position, GQA, keys read through the block table (vLLM learning book
// section 5).
//
// Work item = one workgroup per (sequence, KV head, head chunk, q-tile of BM = 32*RW rows).
// Wave w of the workgroup owns one query head of the KV head's group and 32 rows of the
// tile; all waves share the K/V tiles (64 keys) staged in LDS, so a K/V byte is fetched
// once per q-tile for the whole head group.  Per 64-key tile each wave computes
//   S^T[64 keys x 32 rows] = K . Q^T      (16x16x32 bf16 MFMA, K from LDS, Q^T in VGPRs)
//   online softmax on S^T, P^T packed to bf16 straight from the accumulators
//   O^T[D x 32 rows]   += V^T . P^T        (V^T from LDS)
// V is transposed on its way into LDS: each thread loads one 16-byte chunk (8 dims) of 8
// keys and writes 8 dims x 8 keys with byte permutes.  The 8 keys of a chunk are the ones
// one PV MFMA lane group needs (keys 32c + 16*(j/4) + 4*grp + j%4), so every MFMA operand
// is a single 16-byte LDS read.
//
// Tiles outside the union of the rows' live key ranges are never visited, and keys of a
// visited tile outside that union are zero-filled rather than read, so cache slots outside
// every row's window may hold anything.  Tiles crossing the causal diagonal or the window
// edge get an element mask; interior tiles do not.
//
// Workgroups are numbered so that each XCD (work dispatched round-robin over 8) runs the
// q-tiles of one (sequence, KV head) back to back: those share K/V through that XCD's L2.
#include <math.h>

#include "pa_internal.hpp"

namespace pa {

namespace {

constexpr int BN = 64;  // keys per K/V tile

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    const uint32_t a = __builtin_bit_cast(unsigned short, (__bf16)lo);
    const uint32_t b = __builtin_bit_cast(unsigned short, (__bf16)hi);
    return a | (b << 16);
}
__device__ inline uint32_t dw4(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

}  // namespace

struct PrefillGrid {
    int n_head_chunks;  // workgroups per KV head (heads of the group split in chunks)
    int heads_per_wg;
    int n_sg;           // num_seqs * num_kv_heads * n_head_chunks
    int n_qtiles;       // ceil(max_seqlen_q / BM)
};

template <int D, int RW>
__global__ __launch_bounds__(512) void prefill_bf16_kernel(const PrefillArgs a, const PrefillGrid pg) {
    constexpr int BM = 32 * RW;     // query rows per tile
    constexpr int KS = D / 32;      // k-slices of q.K^T
    constexpr int DB = D / 16;      // 16-dim output blocks
    constexpr int CPR = D / 8;      // 16-byte chunks per K row
    constexpr int KCH = BN * CPR;   // 16-byte chunks per K tile
    constexpr int KIT = KCH / 256;  // chunks per thread (>= 256 threads per workgroup)
    constexpr int VOCT = (BN / 8) * (D / 8);  // 8-key x 8-dim V blocks per tile
    constexpr int KROW = D + 8;     // LDS row stride of K (elements)
    constexpr int VROW = BN + 8;    // LDS row stride of V^T (elements)

    __shared__ __attribute__((aligned(16))) __bf16 lds_k[2][BN * KROW];
    __shared__ __attribute__((aligned(16))) __bf16 lds_v[2][D * VROW];

    // ---------------------------------------------------------------- work item
    const int b = blockIdx.x;
    const int xcd = b & 7;
    const int li = b >> 3;
    const int sg = (li / pg.n_qtiles) * 8 + xcd;
    if (sg >= pg.n_sg) return;
    const int qt = pg.n_qtiles - 1 - li % pg.n_qtiles;  // later (longer) tiles first
    const int per_seq = a.c.num_kv_heads * pg.n_head_chunks;
    const int s = sg / per_seq;
    const int g = (sg % per_seq) / pg.n_head_chunks;
    const int hc = sg % pg.n_head_chunks;

    const int q0 = a.cu_q[s];
    const int sq = a.cu_q[s + 1] - q0;
    const int i0 = qt * BM;
    if (i0 >= sq) return;
    const int sk = a.cu_k[s + 1] - a.cu_k[s];
    const int off = sk - sq;
    const int W = a.window;
    const int rows_end = min(i0 + BM, sq);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int hw = wave / RW;
    const int rw = wave % RW;
    const int hig = hc * pg.heads_per_wg + hw;  // head within the group
    const bool wave_ok = hig < a.group;
    const int h = g * a.group + hig;
    const int H = a.num_heads;
    const int Hkv = a.c.num_kv_heads;

    // key range of the whole tile (union over its rows)
    const int wg_lo = W > 0 ? max(0, off + i0 - W + 1) : 0;
    const int wg_hi = min(off + rows_end - 1, sk - 1);
    // this wave's rows and key range
    const int r0 = i0 + 32 * rw;
    const int r_last = min(r0 + 31, rows_end - 1);
    const bool wave_active = wave_ok && r0 < rows_end;
    const int wv_hi = min(off + r_last, sk - 1);
    const int wv_lo = W > 0 ? max(0, off + r0 - W + 1) : 0;
    const int wv_lo_max = W > 0 ? max(0, off + r_last - W + 1) : 0;
    const int wv_p_min = off + r0;

    const float c_log2 = a.scale * 1.4426950408889634f;
    const int BS = a.c.block_size;
    const int shift = a.c.block_shift;
    const __bf16* kplane = (const __bf16*)a.c.kv;
    const __bf16* vplane = kplane + a.c.plane_elems;
    const int32_t* table = a.table + (int64_t)s * a.max_blocks;

    // ---------------------------------------------------------------- Q^T operands
    bf16x8 qf[2][KS];
    int prow[2], plo[2];
    for (int nb = 0; nb < 2; ++nb) {
        const int row = r0 + 16 * nb + col;
        const bool ok = wave_active && row < rows_end;
        const uint4* src = (const uint4*)((const __bf16*)a.q + ((int64_t)(q0 + row) * H + h) * D);
        for (int t = 0; t < KS; ++t)
            qf[nb][t] = __builtin_bit_cast(bf16x8, ok ? src[4 * t + grp] : make_uint4(0, 0, 0, 0));
        prow[nb] = off + row;
        plo[nb] = W > 0 ? max(0, off + row - W + 1) : 0;
    }

    f32x4 oacc[DB][2];
    for (int d = 0; d < DB; ++d)
        for (int nb = 0; nb < 2; ++nb) oacc[d][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    // ---------------------------------------------------------------- K/V tile staging
    uint4 kreg[KIT];
    uint4 vreg[8];
    const bool v_worker = tid < VOCT;
    // V block of this thread: octet o = (c, gq), dim chunk dc
    const int v_o = tid & 7;
    const int v_dc = tid >> 3;
    const int v_c = v_o >> 2;
    const int v_gq = v_o & 3;

    auto load_tile = [&](int k0) {
        int64_t rowbase[4];
        for (int ga = 0; ga < 4; ++ga) {
            const int j0 = k0 + 16 * ga;
            const bool live = (j0 <= wg_hi) && (j0 + 15 >= wg_lo);
            const int blk = live ? table[j0 >> shift] : 0;
            rowbase[ga] = (int64_t)blk * BS + (j0 & (BS - 1));
        }
        for (int i = 0; i < KIT; ++i) {
            const int c = tid + 256 * i;
            uint4 x = make_uint4(0, 0, 0, 0);
            if (tid < 256) {
                const int kl = c / CPR;
                const int dc = c % CPR;
                const int key = k0 + kl;
                const int ga = kl >> 4;
                const int64_t rb = ga == 0 ? rowbase[0] : ga == 1 ? rowbase[1] : ga == 2 ? rowbase[2] : rowbase[3];
                if (key >= wg_lo && key <= wg_hi)
                    x = *(const uint4*)(kplane + ((rb + (kl & 15)) * Hkv + g) * D + dc * 8);
            }
            kreg[i] = x;
        }
        if (v_worker) {
            for (int j = 0; j < 8; ++j) {
                const int kl = 32 * v_c + 16 * (j >> 2) + 4 * v_gq + (j & 3);
                const int key = k0 + kl;
                const int ga = kl >> 4;
                const int64_t rb = ga == 0 ? rowbase[0] : ga == 1 ? rowbase[1] : ga == 2 ? rowbase[2] : rowbase[3];
                uint4 x = make_uint4(0, 0, 0, 0);
                if (key >= wg_lo && key <= wg_hi)
                    x = *(const uint4*)(vplane + ((rb + (kl & 15)) * Hkv + g) * D + v_dc * 8);
                vreg[j] = x;
            }
        }
    };
    auto store_tile = [&](int buf) {
        if (tid < 256) {
            for (int i = 0; i < KIT; ++i) {
                const int c = tid + 256 * i;
                const int kl = c / CPR;
                const int dc = c % CPR;
                *(uint4*)(&lds_k[buf][kl * KROW + dc * 8]) = kreg[i];
            }
        }
        if (v_worker) {
            const int pos = 32 * v_c + 8 * v_gq;
            for (int e = 0; e < 8; ++e) {
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                const int wsel = e >> 1;
                uint4 w;
                w.x = __builtin_amdgcn_perm(dw4(vreg[1], wsel), dw4(vreg[0], wsel), sel);
                w.y = __builtin_amdgcn_perm(dw4(vreg[3], wsel), dw4(vreg[2], wsel), sel);
                w.z = __builtin_amdgcn_perm(dw4(vreg[5], wsel), dw4(vreg[4], wsel), sel);
                w.w = __builtin_amdgcn_perm(dw4(vreg[7], wsel), dw4(vreg[6], wsel), sel);
                *(uint4*)(&lds_v[buf][(8 * v_dc + e) * VROW + pos]) = w;
            }
        }
    };

    // ---------------------------------------------------------------- one tile of math
    auto compute_tile = [&](int buf, int k0) {
        if (!wave_active || k0 > wv_hi || k0 + BN - 1 < wv_lo) return;
        const bool edge = (k0 + BN - 1 > wv_p_min) || (W > 0 && k0 < wv_lo_max);
        const __bf16* kt = lds_k[buf];
        const __bf16* vt = lds_v[buf];

        f32x4 sacc[4][2];
        for (int ga = 0; ga < 4; ++ga)
            for (int nb = 0; nb < 2; ++nb) sacc[ga][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int t = 0; t < KS; ++t) {
            for (int ga = 0; ga < 4; ++ga) {
                const bf16x8 kf = *(const bf16x8*)(kt + (16 * ga + col) * KROW + 32 * t + 8 * grp);
                for (int nb = 0; nb < 2; ++nb)
                    sacc[ga][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nb][t], sacc[ga][nb], 0, 0, 0);
            }
        }
        if (edge) {
            for (int ga = 0; ga < 4; ++ga)
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + 16 * ga + 4 * grp + r;
                    for (int nb = 0; nb < 2; ++nb)
                        if (key > prow[nb] || key < plo[nb]) sacc[ga][nb][r] = -INFINITY;
                }
        }
        uint4 pk[2][2];  // [32-key chunk][nb]
        bool rescale = false;
        float alpha[2];
        for (int nb = 0; nb < 2; ++nb) {
            float mx = -INFINITY;
            for (int ga = 0; ga < 4; ++ga)
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[ga][nb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[nb], mx * c_log2);
            const float msub = m_new == -INFINITY ? 0.f : m_new;
            alpha[nb] = __builtin_amdgcn_exp2f(m_run[nb] - msub);
            rescale |= (alpha[nb] != 1.f);
            m_run[nb] = m_new;
            float pv[4][4];
            float psum = 0.f;
            for (int ga = 0; ga < 4; ++ga)
                for (int r = 0; r < 4; ++r) {
                    pv[ga][r] = __builtin_amdgcn_exp2f(fmaf(sacc[ga][nb][r], c_log2, -msub));
                    psum += pv[ga][r];
                }
            l_run[nb] = l_run[nb] * alpha[nb] + psum;
            for (int cc = 0; cc < 2; ++cc) {
                pk[cc][nb].x = pack_bf16x2(pv[2 * cc][0], pv[2 * cc][1]);
                pk[cc][nb].y = pack_bf16x2(pv[2 * cc][2], pv[2 * cc][3]);
                pk[cc][nb].z = pack_bf16x2(pv[2 * cc + 1][0], pv[2 * cc + 1][1]);
                pk[cc][nb].w = pack_bf16x2(pv[2 * cc + 1][2], pv[2 * cc + 1][3]);
            }
        }
        if (__any(rescale)) {
            for (int d = 0; d < DB; ++d)
                for (int nb = 0; nb < 2; ++nb) oacc[d][nb] *= alpha[nb];
        }
        for (int d = 0; d < DB; ++d) {
            for (int cc = 0; cc < 2; ++cc) {
                const bf16x8 vf = *(const bf16x8*)(vt + (16 * d + col) * VROW + 32 * cc + 8 * grp);
                for (int nb = 0; nb < 2; ++nb)
                    oacc[d][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        vf, __builtin_bit_cast(bf16x8, pk[cc][nb]), oacc[d][nb], 0, 0, 0);
            }
        }
    };

    // ---------------------------------------------------------------- main loop
    if (wg_hi >= wg_lo) {
        const int kt_begin = wg_lo / BN;
        const int kt_end = wg_hi / BN + 1;
        load_tile(kt_begin * BN);
        store_tile(0);
        __syncthreads();
        for (int kt = kt_begin; kt < kt_end; ++kt) {
            const int buf = (kt - kt_begin) & 1;
            const bool has_next = kt + 1 < kt_end;
            if (has_next) load_tile((kt + 1) * BN);
            compute_tile(buf, kt * BN);
            if (has_next) store_tile(buf ^ 1);
            __syncthreads();
        }
    }

    // ---------------------------------------------------------------- epilogue
    if (!wave_active) return;
    for (int nb = 0; nb < 2; ++nb) {
        float lt = l_run[nb] + __shfl_xor(l_run[nb], 16);
        lt += __shfl_xor(lt, 32);
        const int row = r0 + 16 * nb + col;
        if (row >= rows_end) continue;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        __bf16* dst = (__bf16*)a.out + ((int64_t)(q0 + row) * H + h) * D + 4 * grp;
        for (int d = 0; d < DB; ++d) {
            const f32x4 o = oacc[d][nb];
            *(uint2*)(dst + 16 * d) = make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv),
                                                 pack_bf16x2(o[2] * inv, o[3] * inv));
        }
    }
}

template <int D, int RW>
static void launch_rw(const PrefillArgs& a, const PrefillGrid& pg, int threads, hipStream_t st) {
    const int64_t nsg_pad = ((int64_t)pg.n_sg + 7) / 8 * 8;
    const dim3 grid((unsigned)(nsg_pad * pg.n_qtiles));
    hipLaunchKernelGGL((prefill_bf16_kernel<D, RW>), grid, dim3(threads), 0, st, a, pg);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t st) {
    const int G = a.group;
    // row-waves per head: keep 4..8 waves per workgroup
    const int RW = G >= 4 ? 1 : (G >= 2 ? 2 : 4);
    PrefillGrid pg;
    pg.heads_per_wg = G * RW <= 8 ? G : 8 / RW;
    pg.n_head_chunks = (G + pg.heads_per_wg - 1) / pg.heads_per_wg;
    pg.n_sg = a.num_seqs * a.c.num_kv_heads * pg.n_head_chunks;
    const int BM = 32 * RW;
    pg.n_qtiles = (a.max_seqlen_q + BM - 1) / BM;
    const int threads = 64 * RW * pg.heads_per_wg < 256 ? 256 : 64 * RW * pg.heads_per_wg;
    if (a.c.head_size == 128) {
        if (RW == 1) launch_rw<128, 1>(a, pg, threads, st);
        else if (RW == 2) launch_rw<128, 2>(a, pg, threads, st);
        else launch_rw<128, 4>(a, pg, threads, st);
    } else {
        if (RW == 1) launch_rw<64, 1>(a, pg, threads, st);
        else if (RW == 2) launch_rw<64, 2>(a, pg, threads, st);
        else launch_rw<64, 4>(a, pg, threads, st);
    }
    return hipGetLastError();
}

}  // namespace pa
