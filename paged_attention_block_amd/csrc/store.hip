// KV store scatter and block copies: bitwise moves of 16-byte chunks (and the quantizing
// store of an FP8 cache).
//
// Store (MinivLLM API docs, "Attention", store_kvcache; vLLM learning book section 10 Q2):
// the flat slot index equals the row index of the [NB*BS] token rows of a cache plane, so a
// token's destination row is simply `slot`, with no division.  A workgroup takes a few
// consecutive tokens; its threads cover the K and V rows in consecutive 16-byte chunks, so
// every wave writes whole contiguous rows (2 KB per plane for 8 KV heads x 128 bf16).
#include "pa_internal.hpp"

namespace pa {

// Holds every chunk of a batch until its load has arrived: one wait after all the loads
// of the batch are in flight, instead of the compiler sinking each load into its store's
// branch, where it waits for that load alone.  (Two tokens per workgroup measure 10% faster
// than one on a 13894-token store; four are no faster, eight slower.)
template <int N>
__device__ inline void hold(u32x4 (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}

template <int TPW>
__global__ __launch_bounds__(256) void store_kernel(u32x4* __restrict__ cache,
                                                    const u32x4* __restrict__ key,
                                                    const u32x4* __restrict__ value,
                                                    const int32_t* __restrict__ slots,
                                                    int32_t num_tokens, int32_t row_chunks,
                                                    int64_t plane_chunks) {
    // TPW tokens per workgroup: a thread issues the loads of its chunk of every token before
    // the first store, so each thread keeps TPW 16-byte reads in flight.  A token past the
    // end reads the last token's row, and a token with a negative slot is read but not
    // stored.
    const int32_t t0 = blockIdx.x * TPW;
    int32_t slot[TPW];
    int64_t row[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        slot[i] = t0 + i < num_tokens ? slots[t0 + i] : -1;
        row[i] = (int64_t)min(t0 + i, num_tokens - 1) * row_chunks;
    }
    for (int32_t c = threadIdx.x; c < 2 * row_chunks; c += blockDim.x) {
        const bool is_v = c >= row_chunks;
        const int32_t cc = is_v ? c - row_chunks : c;
        const u32x4* src = is_v ? value : key;
        u32x4* dst = cache + (is_v ? plane_chunks : 0) + cc;
        u32x4 x[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) x[i] = src[row[i] + cc];
        hold(x);
#pragma unroll
        for (int i = 0; i < TPW; ++i)
            if (slot[i] >= 0) dst[(int64_t)slot[i] * row_chunks] = x[i];
    }
}

// FP8 (E4M3) cache: a thread turns one 16-byte piece of a bf16 key or value row (8 elements)
// into 8 cache bytes, e4m3(x * r) with r = fp32(1 / kv_scale): the product in fp32,
// magnitudes above 448 saturated (NaN passes through), then v_cvt_pk_fp8_f32 (round to
// nearest even) two elements at a time.
__device__ inline float sat_e4m3(float x) { return fabsf(x) > 448.f ? copysignf(448.f, x) : x; }
__device__ inline uint32_t e4m3x4(uint32_t lo, uint32_t hi, float r) {
    // lo, hi: two bf16 pairs (element 2i in the low half)
    const float a = __uint_as_float(lo << 16) * r, b = __uint_as_float(lo & 0xffff0000u) * r;
    const float c = __uint_as_float(hi << 16) * r, d = __uint_as_float(hi & 0xffff0000u) * r;
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), (int)w, true);
}

template <int TPW>
__global__ __launch_bounds__(256) void store_fp8_kernel(u32x2* __restrict__ cache,
                                                        const u32x4* __restrict__ key,
                                                        const u32x4* __restrict__ value,
                                                        const int32_t* __restrict__ slots,
                                                        int32_t num_tokens, int32_t row_chunks,
                                                        int64_t plane_chunks, float r) {
    // row_chunks: 16-byte pieces of an input row = 8-byte pieces of a cache row.  TPW tokens
    // per workgroup, loads first, as in store_kernel.
    const int32_t t0 = blockIdx.x * TPW;
    int32_t slot[TPW];
    int64_t row[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        slot[i] = t0 + i < num_tokens ? slots[t0 + i] : -1;
        row[i] = (int64_t)min(t0 + i, num_tokens - 1) * row_chunks;
    }
    for (int32_t c = threadIdx.x; c < 2 * row_chunks; c += blockDim.x) {
        const bool is_v = c >= row_chunks;
        const int32_t cc = is_v ? c - row_chunks : c;
        const u32x4* src = is_v ? value : key;
        u32x2* dst = cache + (is_v ? plane_chunks : 0) + cc;
        u32x4 x[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) x[i] = src[row[i] + cc];
        hold(x);
#pragma unroll
        for (int i = 0; i < TPW; ++i)
            if (slot[i] >= 0)
                dst[(int64_t)slot[i] * row_chunks] = u32x2{e4m3x4(x[i][0], x[i][1], r), e4m3x4(x[i][2], x[i][3], r)};
    }
}

// copy_blocks (vllm-npu 0.4.2 diff, backend copy_blocks): one workgroup per (pair, plane),
// each moving the block's BS*Hkv*D elements as 16-byte chunks.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int32_t block_chunks,
                                                          int64_t plane_chunks) {
    const int32_t pair = blockIdx.x >> 1;
    const int32_t plane = blockIdx.x & 1;
    const int64_t src = (int64_t)pairs[2 * pair] * block_chunks + plane * plane_chunks;
    const int64_t dst = (int64_t)pairs[2 * pair + 1] * block_chunks + plane * plane_chunks;
    for (int32_t c = threadIdx.x; c < block_chunks; c += blockDim.x) cache[dst + c] = cache[src + c];
}

hipError_t launch_store(const StoreArgs& a, hipStream_t s) {
    if (a.c.dtype == 2) {
        const int32_t row_chunks = a.c.num_kv_heads * a.c.head_size / 8;
        const int64_t plane_chunks = a.c.plane_elems / 8;
        int threads = 2 * row_chunks;
        threads = threads > 256 ? 256 : ((threads + 63) / 64) * 64;
        constexpr int kTpw = 2;
        hipLaunchKernelGGL(store_fp8_kernel<kTpw>, dim3((int32_t)(((int64_t)a.num_tokens + kTpw - 1) / kTpw)),
                           dim3(threads), 0, s, (u32x2*)a.c.kv, (const u32x4*)a.key, (const u32x4*)a.value,
                           a.slots, a.num_tokens, row_chunks, plane_chunks, a.c.kv_inv_scale);
        return hipGetLastError();
    }
    const int elt = cache_elt(a.c.dtype);
    const int32_t row_chunks = a.c.num_kv_heads * a.c.head_size * elt / 16;
    const int64_t plane_chunks = a.c.plane_elems * elt / 16;
    int threads = 2 * row_chunks;
    threads = threads > 256 ? 256 : ((threads + 63) / 64) * 64;
    constexpr int kTpw = 2;
    hipLaunchKernelGGL(store_kernel<kTpw>, dim3((int32_t)(((int64_t)a.num_tokens + kTpw - 1) / kTpw)),
                       dim3(threads), 0, s, (u32x4*)a.c.kv, (const u32x4*)a.key, (const u32x4*)a.value, a.slots,
                       a.num_tokens, row_chunks, plane_chunks);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t s) {
    const int elt = cache_elt(a.c.dtype);
    const int32_t block_chunks =
        (int32_t)((int64_t)a.c.block_size * a.c.num_kv_heads * a.c.head_size * elt / 16);
    const int64_t plane_chunks = a.c.plane_elems * elt / 16;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(2 * a.num_pairs), dim3(256), 0, s,
                       (uint4*)a.c.kv, a.pairs, block_chunks, plane_chunks);
    return hipGetLastError();
}

}  // namespace pa
