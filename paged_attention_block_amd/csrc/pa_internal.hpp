// Internal declarations shared by the HIP translation units of libpa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---------------------------------------------------------------- device vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Lanes of one wavefront.
constexpr int kWave = 64;

// Split-K bookkeeping for decode.  A sequence with n keys and window lower bound lo is cut
// into partitions of `part` keys (a multiple of 64) starting at lo rounded down to 32, so
// every 32-key step is aligned in absolute key index.
__host__ __device__ inline int decode_base(int lo) { return lo & ~31; }
__host__ __device__ inline int decode_lo(int n, int window) {
    return (window > 0 && n > window) ? n - window : 0;
}
__host__ __device__ inline int decode_num_parts(int n, int window, int part) {
    if (n <= 0) return 0;
    int base = decode_base(decode_lo(n, window));
    return (n - base + part - 1) / part;
}

// ---------------------------------------------------------------- launch parameter blocks
struct CacheArgs {
    void* kv;            // [2][NB][BS][Hkv][D]
    int64_t plane_elems; // NB*BS*Hkv*D
    int32_t num_blocks;
    int32_t block_size;
    int32_t block_shift; // log2(block_size)
    int32_t num_kv_heads;
    int32_t head_size;
    int32_t dtype;       // 0 f32, 1 bf16
};

struct StoreArgs {
    CacheArgs c;
    const void* key;
    const void* value;
    const int32_t* slots;
    int32_t num_tokens;
};

struct CopyArgs {
    CacheArgs c;
    const int32_t* pairs;
    int32_t num_pairs;
};

struct PrefillArgs {
    CacheArgs c;
    void* out;
    const void* q;
    const int32_t* table;
    int32_t max_blocks;
    const int32_t* cu_q;
    const int32_t* cu_k;
    int32_t num_seqs;
    int32_t max_seqlen_q;
    int32_t num_heads;
    int32_t group;       // num_heads / num_kv_heads
    float scale;
    int32_t window;
};

struct DecodeArgs {
    CacheArgs c;
    void* out;
    const void* q;
    const int32_t* table;
    int32_t max_blocks;
    const int32_t* seq_lens;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t group;
    float scale;
    int32_t window;
    int32_t part;        // keys per partition (multiple of 64)
    int32_t max_parts;   // partitions per sequence the workspace holds
    float* ws_o;         // [B][H][max_parts][D] unnormalised partial outputs
    float* ws_ml;        // [B][H][max_parts][2] running max (log2 units) and sum
};

// Host launchers (return hipGetLastError() of the launches).
hipError_t launch_store(const StoreArgs& a, hipStream_t s);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace pa
