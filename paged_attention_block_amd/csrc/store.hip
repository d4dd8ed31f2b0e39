// KV store scatter and block copies: bitwise moves of 16-byte chunks.
//
// Store (MinivLLM API docs, "Attention", store_kvcache; vLLM learning book section 10 Q2):
// the flat slot index equals the row index of the [NB*BS] token rows of a cache plane, so a
// token's destination row is simply `slot`, with no division.  One workgroup per token:
// threads cover the K and V rows in consecutive 16-byte chunks, so every wave writes whole
// contiguous rows (2 KB per plane for 8 KV heads x 128 bf16).
#include "pa_internal.hpp"

namespace pa {

__global__ __launch_bounds__(256) void store_kernel(uint4* __restrict__ cache,
                                                    const uint4* __restrict__ key,
                                                    const uint4* __restrict__ value,
                                                    const int32_t* __restrict__ slots,
                                                    int32_t row_chunks, int64_t plane_chunks) {
    const int32_t t = blockIdx.x;
    const int32_t slot = slots[t];
    if (slot < 0) return;
    const int64_t src = (int64_t)t * row_chunks;
    const int64_t dst = (int64_t)slot * row_chunks;
    for (int32_t c = threadIdx.x; c < 2 * row_chunks; c += blockDim.x) {
        const bool is_v = c >= row_chunks;
        const int32_t cc = is_v ? c - row_chunks : c;
        const uint4 x = is_v ? value[src + cc] : key[src + cc];
        cache[(is_v ? plane_chunks : 0) + dst + cc] = x;
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
    const int elt = a.c.dtype == 1 ? 2 : 4;
    const int32_t row_chunks = a.c.num_kv_heads * a.c.head_size * elt / 16;
    const int64_t plane_chunks = a.c.plane_elems * elt / 16;
    int threads = 2 * row_chunks;
    threads = threads > 256 ? 256 : ((threads + 63) / 64) * 64;
    hipLaunchKernelGGL(store_kernel, dim3(a.num_tokens), dim3(threads), 0, s,
                       (uint4*)a.c.kv, (const uint4*)a.key, (const uint4*)a.value, a.slots,
                       row_chunks, plane_chunks);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t s) {
    const int elt = a.c.dtype == 1 ? 2 : 4;
    const int32_t block_chunks =
        (int32_t)((int64_t)a.c.block_size * a.c.num_kv_heads * a.c.head_size * elt / 16);
    const int64_t plane_chunks = a.c.plane_elems * elt / 16;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(2 * a.num_pairs), dim3(256), 0, s,
                       (uint4*)a.c.kv, a.pairs, block_chunks, plane_chunks);
    return hipGetLastError();
}

}  // namespace pa
