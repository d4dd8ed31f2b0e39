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
// V is transposed on its way into LDS: a thread loads one 16-byte chunk (8 dims) of 8 keys
// and writes 8 dims x 8 keys with byte permutes.  The 8 keys of a chunk are the ones one
// PV MFMA lane group needs (keys 32c + 16*(j/4) + 4*grp + j%4), so every MFMA operand is a
// single 16-byte LDS read.  LDS rows are padded by 16 bytes, which keeps the 16 lanes that
// read 16 different rows on distinct banks.
//
// Tiles outside the union of the rows' live key ranges are never visited; inside a
// visited tile, keys outside that union are loaded from a live block of the same tile
// (never through an unread block-table entry) and zeroed before they reach LDS, so cache
// slots outside every row's window may hold anything.  Tiles crossing the causal diagonal
// or the window edge get an element mask; interior tiles do not.
//
// Workgroups are numbered so that each XCD (work dispatched round-robin over 8) runs the
// q-tiles of one (sequence, KV head) back to back: those share K/V through that XCD's L2.
#include <math.h>

#include "pa_internal.hpp"

namespace pa {

namespace {
constexpr int BN = 64;  // keys per K/V tile
}  // namespace

struct PrefillGrid {
    int n_head_chunks;  // workgroups per KV head (heads of the group split in chunks)
    int heads_per_wg;
    int n_sg;           // num_seqs * num_kv_heads * n_head_chunks
    int n_qtiles;       // ceil(max_seqlen_q / BM)
};

template <int D, int RW>
__global__ __launch_bounds__(512) void prefill_bf16_kernel(const PrefillArgs a, const PrefillGrid pg) {
    constexpr int BM = 32 * RW;       // query rows per tile
    constexpr int KS = D / 32;        // k-slices of q.K^T
    constexpr int DB = D / 16;        // 16-dim output blocks
    constexpr int CPR = D / 8;        // 16-byte chunks per K row
    constexpr int KIT = BN * CPR / 256;   // K chunks per staging thread (threads 0..255)
    constexpr int KRPI = 256 / CPR;       // K rows per staging round
    constexpr int VOCT = (BN / 8) * (D / 8);  // 8-key x 8-dim V blocks per tile
    constexpr int KROW = D + 8;       // LDS row stride of K (elements)
    constexpr int VROW = BN + 8;      // LDS row stride of V^T (elements)

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
    const char* __restrict__ kplane = (const char*)a.c.kv;
    const char* __restrict__ vplane = kplane + a.c.plane_elems * 2;
    const int32_t* __restrict__ table = a.table + (int64_t)s * a.max_blocks;
    const int64_t RB = (int64_t)Hkv * D * 2;  // cache token-row bytes

    // ---------------------------------------------------------------- Q^T operands
    bf16x8 qf[2][KS];
    int prow[2], plo[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int row = r0 + 16 * nb + col;
        const bool ok = wave_active && row < rows_end;
        const u32x4* src = (const u32x4*)((const __bf16*)a.q + ((int64_t)(q0 + (ok ? row : 0)) * H + (wave_ok ? h : 0)) * D);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const u32x4 x = src[4 * t + grp];
            qf[nb][t] = __builtin_bit_cast(bf16x8, ok ? x : (u32x4)(0u));
        }
        prow[nb] = off + row;
        plo[nb] = W > 0 ? max(0, off + row - W + 1) : 0;
    }

    f32x4 oacc[DB][2];
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) oacc[d][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    // ---------------------------------------------------------------- K/V tile staging
    // K: thread tid < 256 stages chunks (row k_r0 + KRPI*i, column k_dc), i < KIT; the row's
    // 16-key group is (k_r0 >> 4) + (KRPI / 16) * i, uniform within a wave.
    const bool k_worker = tid < 256;
    const int k_r0 = tid / CPR;
    const int k_dc = tid - k_r0 * CPR;
    const uint32_t k_goff = (uint32_t)((((k_r0 & 15) * Hkv + g) * D + k_dc * 8) * 2);
    const uint32_t k_loff = (uint32_t)(k_r0 * KROW + k_dc * 8);
    // V: thread tid < VOCT stages the 8 keys 32*v_c + 16*(j/4) + 4*v_gq + j%4 at dims
    // 8*v_dc .. +8 (rows 4*v_gq + j%4 of groups 2*v_c + j/4)
    const bool v_worker = tid < VOCT;
    const int v_o = tid & 7;
    const int v_dc = tid >> 3;
    const int v_c = v_o >> 2;
    const int v_gq = v_o & 3;
    const uint32_t v_goff = (uint32_t)((((4 * v_gq) * Hkv + g) * D + v_dc * 8) * 2);
    const uint32_t v_loff = (uint32_t)(8 * v_dc * VROW + 32 * v_c + 8 * v_gq);

    u32x4 kreg[KIT];
    u32x4 vreg[8];

    auto load_tile = [&](int k0) {
        int64_t gb[4];
        bool gv[4];
#pragma unroll
        for (int ga = 0; ga < 4; ++ga) {
            const int j0 = k0 + 16 * ga;
            gv[ga] = (j0 <= wg_hi) && (j0 + 15 >= wg_lo);
            const int blk = gv[ga] ? table[j0 >> shift] : 0;
            gb[ga] = ((int64_t)blk * BS + (j0 & (BS - 1))) * RB;
        }
        // a group with no live key borrows the rows of a live group of the tile
        const int64_t live = gv[0] ? gb[0] : gv[1] ? gb[1] : gv[2] ? gb[2] : gb[3];
#pragma unroll
        for (int ga = 0; ga < 4; ++ga) gb[ga] = gv[ga] ? gb[ga] : live;
        if (k_worker) {
#pragma unroll
            for (int i = 0; i < KIT; ++i) {
                const int ga = (k_r0 >> 4) + (KRPI / 16) * i;
                const int64_t base = ga == 0 ? gb[0] : ga == 1 ? gb[1] : ga == 2 ? gb[2] : gb[3];
                kreg[i] = *(const u32x4*)(kplane + base + k_goff);
            }
        }
        if (v_worker) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t base = v_c ? gb[2 + (j >> 2)] : gb[j >> 2];
                vreg[j] = *(const u32x4*)(vplane + base + v_goff + (j & 3) * RB);
            }
        }
    };
    auto store_tile = [&](int buf, int k0) {
        const bool zero = (k0 < wg_lo) || (k0 + BN - 1 > wg_hi);
        if (k_worker) {
#pragma unroll
            for (int i = 0; i < KIT; ++i) {
                u32x4 x = kreg[i];
                if (zero) {
                    const int key = k0 + k_r0 + KRPI * i;
                    x = (key >= wg_lo && key <= wg_hi) ? x : (u32x4)(0u);
                }
                *(u32x4*)(&lds_k[buf][k_loff + KRPI * i * KROW]) = x;
            }
        }
        if (v_worker) {
            if (zero) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int key = k0 + 32 * v_c + 16 * (j >> 2) + 4 * v_gq + (j & 3);
                    vreg[j] = (key >= wg_lo && key <= wg_hi) ? vreg[j] : (u32x4)(0u);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                const int ws = e >> 1;
                u32x4 w;
                w[0] = __builtin_amdgcn_perm(vreg[1][ws], vreg[0][ws], sel);
                w[1] = __builtin_amdgcn_perm(vreg[3][ws], vreg[2][ws], sel);
                w[2] = __builtin_amdgcn_perm(vreg[5][ws], vreg[4][ws], sel);
                w[3] = __builtin_amdgcn_perm(vreg[7][ws], vreg[6][ws], sel);
                *(u32x4*)(&lds_v[buf][v_loff + e * VROW]) = w;
            }
        }
    };

    // LDS operand offsets of this lane (elements)
    const int kop = col * KROW + 8 * grp;
    const int vop = col * VROW + 8 * grp;

    // ---------------------------------------------------------------- one tile of math
    auto compute_tile = [&](int buf, int k0) {
        if (!wave_active || k0 > wv_hi || k0 + BN - 1 < wv_lo) return;
        const bool edge = (k0 + BN - 1 > wv_p_min) || (W > 0 && k0 < wv_lo_max);
        const __bf16* kt = lds_k[buf] + kop;
        const __bf16* vt = lds_v[buf] + vop;

        f32x4 sacc[4][2];
#pragma unroll
        for (int ga = 0; ga < 4; ++ga)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) sacc[ga][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KS; ++t) {
#pragma unroll
            for (int ga = 0; ga < 4; ++ga) {
                const bf16x8 kf = *(const bf16x8*)(kt + 16 * ga * KROW + 32 * t);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    sacc[ga][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nb][t], sacc[ga][nb], 0, 0, 0);
            }
        }
        if (edge) {
#pragma unroll
            for (int ga = 0; ga < 4; ++ga)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + 16 * ga + 4 * grp + r;
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        sacc[ga][nb][r] = (key > prow[nb] || key < plo[nb]) ? -INFINITY : sacc[ga][nb][r];
                }
        }
        u32x4 pk[2][2];  // [32-key chunk][nb]
        float alpha[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            float mx = fmaxf(fmaxf(sacc[0][nb][0], sacc[0][nb][1]), fmaxf(sacc[0][nb][2], sacc[0][nb][3]));
#pragma unroll
            for (int ga = 1; ga < 4; ++ga)
                mx = fmaxf(mx, fmaxf(fmaxf(sacc[ga][nb][0], sacc[ga][nb][1]), fmaxf(sacc[ga][nb][2], sacc[ga][nb][3])));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[nb], mx * c_log2);
            const float msub = m_new == -INFINITY ? 0.f : m_new;
            alpha[nb] = __builtin_amdgcn_exp2f(m_run[nb] - msub);
            m_run[nb] = m_new;
            float pv[4][4];
            float ps[4];
#pragma unroll
            for (int ga = 0; ga < 4; ++ga) {
#pragma unroll
                for (int r = 0; r < 4; ++r) pv[ga][r] = __builtin_amdgcn_exp2f(fmaf(sacc[ga][nb][r], c_log2, -msub));
                ps[ga] = (pv[ga][0] + pv[ga][1]) + (pv[ga][2] + pv[ga][3]);
            }
            l_run[nb] = l_run[nb] * alpha[nb] + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                pk[cc][nb][0] = pack_bf16x2(pv[2 * cc][0], pv[2 * cc][1]);
                pk[cc][nb][1] = pack_bf16x2(pv[2 * cc][2], pv[2 * cc][3]);
                pk[cc][nb][2] = pack_bf16x2(pv[2 * cc + 1][0], pv[2 * cc + 1][1]);
                pk[cc][nb][3] = pack_bf16x2(pv[2 * cc + 1][2], pv[2 * cc + 1][3]);
            }
        }
        if (__any(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
            for (int d = 0; d < DB; ++d)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) oacc[d][nb] *= alpha[nb];
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                const bf16x8 vf = *(const bf16x8*)(vt + 16 * d * VROW + 32 * cc);
#pragma unroll
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
        store_tile(0, kt_begin * BN);
        __syncthreads();
        for (int kt = kt_begin; kt < kt_end; ++kt) {
            const int buf = (kt - kt_begin) & 1;
            const bool has_next = kt + 1 < kt_end;
            if (has_next) load_tile((kt + 1) * BN);
            compute_tile(buf, kt * BN);
            if (has_next) store_tile(buf ^ 1, (kt + 1) * BN);
            __syncthreads();
        }
    }

    // ---------------------------------------------------------------- epilogue
    if (!wave_active) return;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        float lt = l_run[nb] + __shfl_xor(l_run[nb], 16);
        lt += __shfl_xor(lt, 32);
        const int row = r0 + 16 * nb + col;
        if (row >= rows_end) continue;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        __bf16* dst = (__bf16*)a.out + ((int64_t)(q0 + row) * H + h) * D + 4 * grp;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
            const f32x4 o = oacc[d][nb];
            *(u32x2*)(dst + 16 * d) = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
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
