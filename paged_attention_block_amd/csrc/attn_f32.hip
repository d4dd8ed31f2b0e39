// float32 paged attention (prefill and decode) on the vector ALU.
//
// The float32 path exists for exactness checks at small sizes (tolerance 1e-5), so it stays
// simple: one wavefront per (query row, head); lane l owns dims l and l + 64.  For each key
// in the row's live range the wave reads the K row through the block table, reduces q.k
// across lanes, updates the online-softmax state (MinivLLM API docs, "Attention":
// online softmax) and accumulates p * V.  With ALiBi slopes the score of key j at query
// position p gets slope * (j - p) added after the scale (vllm-npu 0.4.2 diff, torch_sdpa.py,
// _make_alibi_bias).  No float32 input ever passes through a bf16 or
// reduced-precision matrix instruction.
#include <math.h>

#include "pa_internal.hpp"

namespace pa {

namespace {
__device__ inline float wave_sum_f32(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
}  // namespace

// mode 0: prefill (blockIdx.x = s * max_seqlen_q + row), mode 1: decode (blockIdx.x = s).
template <int D>
__global__ __launch_bounds__(64) void attn_rows_f32_kernel(
    const float* __restrict__ kv, int64_t plane_elems, int block_size, int block_shift,
    int num_kv_heads, float* __restrict__ out, const float* __restrict__ q,
    const int32_t* __restrict__ table, int max_blocks, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ seq_lens, int max_seqlen_q,
    int num_heads, int group, float scale, int window, const float* __restrict__ alibi, int mode) {
    constexpr int R = D / 64;
    const int lane = threadIdx.x;
    const int h = blockIdx.y;
    int s, token, lo, hi, pos;
    if (mode == 0) {
        s = blockIdx.x / max_seqlen_q;
        const int row = blockIdx.x % max_seqlen_q;
        const int q0 = cu_q[s];
        const int sq = cu_q[s + 1] - q0;
        if (row >= sq) return;
        const int sk = cu_k[s + 1] - cu_k[s];
        const int p = sk - sq + row;
        token = q0 + row;
        pos = p;
        hi = min(p, sk - 1);
        lo = window > 0 ? max(0, p - window + 1) : 0;
    } else {
        s = blockIdx.x;
        token = s;
        const int n = seq_lens[s];
        hi = n - 1;
        pos = n - 1;
        lo = window > 0 ? max(0, n - window) : 0;
    }
    const float slope = alibi ? alibi[h] : 0.f;  // ALiBi: slope * (j - pos) after the scale
    const int g = h / group;
    float qv[R], o[R];
    for (int r = 0; r < R; ++r) {
        qv[r] = q[((int64_t)token * num_heads + h) * D + lane + 64 * r];
        o[r] = 0.f;
    }
    const int32_t* trow = table + (int64_t)s * max_blocks;
    float m = -INFINITY, l = 0.f;
    for (int j = lo; j <= hi; ++j) {
        const int64_t row = (int64_t)trow[j >> block_shift] * block_size + (j & (block_size - 1));
        const float* k = kv + (row * num_kv_heads + g) * D;
        const float* v = k + plane_elems;
        float part = 0.f;
        for (int r = 0; r < R; ++r) part = fmaf(qv[r], k[lane + 64 * r], part);
        const float z = fmaf(wave_sum_f32(part), scale, slope * (float)(j - pos));
        const float m_new = fmaxf(m, z);
        const float alpha = expf(m - m_new);
        const float pj = expf(z - m_new);
        l = l * alpha + pj;
        for (int r = 0; r < R; ++r) o[r] = fmaf(pj, v[lane + 64 * r], o[r] * alpha);
        m = m_new;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    for (int r = 0; r < R; ++r) out[((int64_t)token * num_heads + h) * D + lane + 64 * r] = o[r] * inv;
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)a.num_seqs * a.max_seqlen_q), a.num_heads);
    const CacheArgs& c = a.c;
    if (c.head_size == 128)
        hipLaunchKernelGGL(attn_rows_f32_kernel<128>, grid, dim3(64), 0, st, (const float*)c.kv,
                           c.plane_elems, c.block_size, c.block_shift, c.num_kv_heads,
                           (float*)a.out, (const float*)a.q, a.table, a.max_blocks, a.cu_q, a.cu_k,
                           (const int32_t*)nullptr, a.max_seqlen_q, a.num_heads, a.group, a.scale,
                           a.window, a.alibi, 0);
    else
        hipLaunchKernelGGL(attn_rows_f32_kernel<64>, grid, dim3(64), 0, st, (const float*)c.kv,
                           c.plane_elems, c.block_size, c.block_shift, c.num_kv_heads,
                           (float*)a.out, (const float*)a.q, a.table, a.max_blocks, a.cu_q, a.cu_k,
                           (const int32_t*)nullptr, a.max_seqlen_q, a.num_heads, a.group, a.scale,
                           a.window, a.alibi, 0);
    return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t st) {
    const dim3 grid(a.num_seqs, a.num_heads);
    const CacheArgs& c = a.c;
    if (c.head_size == 128)
        hipLaunchKernelGGL(attn_rows_f32_kernel<128>, grid, dim3(64), 0, st, (const float*)c.kv,
                           c.plane_elems, c.block_size, c.block_shift, c.num_kv_heads,
                           (float*)a.out, (const float*)a.q, a.table, a.max_blocks,
                           (const int32_t*)nullptr, (const int32_t*)nullptr, a.seq_lens, 1,
                           a.num_heads, a.group, a.scale, a.window, a.alibi, 1);
    else
        hipLaunchKernelGGL(attn_rows_f32_kernel<64>, grid, dim3(64), 0, st, (const float*)c.kv,
                           c.plane_elems, c.block_size, c.block_shift, c.num_kv_heads,
                           (float*)a.out, (const float*)a.q, a.table, a.max_blocks,
                           (const int32_t*)nullptr, (const int32_t*)nullptr, a.seq_lens, 1,
                           a.num_heads, a.group, a.scale, a.window, a.alibi, 1);
    return hipGetLastError();
}

}  // namespace pa
