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

// Reductions over the four lanes l, l^16, l^32, l^48 (the four 16-lane groups), with the
// register-only lane swaps of gfx950: permlane16_swap(v, v) yields v of lanes l and l^16
// (in some order), permlane32_swap(v, v) those of l and l^32.
__device__ inline float group4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
    v = fmaxf(__builtin_bit_cast(float, (unsigned)a[0]), __builtin_bit_cast(float, (unsigned)a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}
__device__ inline float group4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
    v = __builtin_bit_cast(float, (unsigned)a[0]) + __builtin_bit_cast(float, (unsigned)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
    return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
}

// Two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Lanes of one wavefront.
constexpr int kWave = 64;

// Split-K bookkeeping for decode.  Sequence s with n keys attends [lo, n); its keys are
// walked in 32-key steps from lo rounded down to 32, so every step is aligned in absolute
// key index.  The steps of the whole batch, sequence after sequence, form one list that is
// cut into equal chunks, one per partition workgroup.  `start` > 0 (shared-prefix decode)
// leaves keys [0, start) to the prefix pass: lo is then at least start.
__host__ __device__ inline int decode_base(int lo) { return lo & ~31; }
__host__ __device__ inline int decode_lo(int n, int window, int start) {
    const int lo = (window > 0 && n > window) ? n - window : 0;
    return lo > start ? lo : start;
}
__host__ __device__ inline int decode_steps(int n, int window, int start) {
    const int lo = decode_lo(n, window, start);
    return n > lo ? (n - decode_base(lo) + 31) >> 5 : 0;
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
    int32_t dtype;       // 0 f32, 1 bf16, 2 fp8 e4m3 (q/k/v/out bf16)
    float kv_scale;      // fp8: the cache holds value / kv_scale (1 otherwise)
    float kv_inv_scale;  // fp8: fp32(1 / kv_scale), the store's multiplier
};

// Bytes per cache element.
__host__ __device__ inline int cache_elt(int dtype) { return dtype == 0 ? 4 : (dtype == 1 ? 2 : 1); }

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
    // fused store (null when the call only attends): the new tokens' keys and values,
    // [tokens][Hkv][D] in query-row order, and their slots.  Keys at positions >= seqlen_k -
    // seqlen_q of a sequence are its new tokens: they are read from here, and written to the
    // cache at their slots by the kernel.
    const void* knew;
    const void* vnew;
    const int32_t* slots;
    const float* alibi;  // [num_heads] ALiBi slopes, or null
    // shared-prefix pass (the prefix instantiation only): the queries are the num_seqs x
    // num_heads decode queries, the keys chunk c of [0, prefix_len) read through table row 0,
    // no causal mask; each (chunk, query row, head) leaves its state in pre_o / pre_ml
    int32_t prefix_len;
    int32_t prefix_chunks;
    float* pre_o;        // [prefix_chunks][num_seqs][H][D]
    float* pre_ml;       // [prefix_chunks][num_seqs][H][2]
    // shared-prefix prefill (cascade != 0): every sequence's keys [0, prefix_len) are one
    // shared prefix, already attended by the prefix pass for all prefix_rows packed query rows
    // (states in pre_o / pre_ml, indexed by packed row); this call attends keys from
    // prefix_len on and folds those states in
    int32_t cascade;
    int32_t prefix_rows;
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
    int32_t nw;          // chunk workgroups per group of 8 KV heads (grid x)
    int32_t min_steps;   // fewest 32-key steps per chunk
    const float* alibi;  // [num_heads] ALiBi slopes, or null
    float* ws_o;         // [nw][2][H][D] unnormalised partial outputs (first, last segment)
    float* ws_ml;        // [nw][2][H][2] running max (log2 units) and sum
    // shared-prefix decode: every sequence's keys [0, key_start) are one shared prefix,
    // attended by the prefix pass in prefix_chunks key chunks whose states (unnormalised
    // output; running max in log2 units and sum) the partition kernel folds in
    int32_t key_start;
    int32_t prefix_chunks;
    int32_t prefix_mfma; // 1: the prefix pass runs on the prefill kernel, 0: the split-key kernel
    float* pre_o;        // [prefix_chunks][num_seqs][H][D]
    float* pre_ml;       // [prefix_chunks][num_seqs][H][2]
    // decode with the store fused (bf16 cache): each sequence's new token, its key n - 1, is
    // read from knew / vnew ([num_seqs][Hkv][D]) instead of the cache, and written to cache slot
    // slots[s] (negative: not written) by the workgroup holding that key; null knew: no store
    const void* knew;
    const void* vnew;
    const int32_t* slots;
};

// Host launchers (return hipGetLastError() of the launches).
hipError_t launch_store(const StoreArgs& a, hipStream_t s);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
// Shared-prefix decode (bf16): prefix pass, then the partition (+ merge) kernels.
hipError_t launch_cascade_decode_bf16(const DecodeArgs& a, hipStream_t s);
// The prefix pass of shared-prefix decode on the prefill kernel: the decode queries of the
// batch against the prefix chunks, states into a.pre_o / a.pre_ml.
hipError_t launch_prefix_states(const DecodeArgs& a, hipStream_t s);
// The prefix pass alone (prefill kernel or split-key kernel, by a.prefix_mfma): the a.num_seqs
// query rows of a.q against the shared prefix [0, a.key_start), states into a.pre_o / a.pre_ml.
hipError_t launch_prefix_pass(const DecodeArgs& a, hipStream_t s);
// 64-key tiles of the prefill kernel's prefix pass per chunk, and its workgroups per chunk.
int prefix_tiles(int prefix_len);
int prefix_workgroups_per_chunk(int num_seqs, int group, int num_kv_heads);
// Partition workgroups of the bf16 decode kernel that fit on the current device at once
// (compute units x resident workgroups per unit); 256 when the device cannot be queried.
int decode_resident_slots(int head_size, int num_kv_heads);

}  // namespace pa
