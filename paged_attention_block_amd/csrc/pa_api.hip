// C ABI of libpa: host-side argument checks, launch planning and dispatch.
//
// Every scalar is validated before the first HIP call, so a rejected call touches no
// device state.  The library never allocates memory and never synchronises: calls only
// enqueue kernels on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "pa.h"
#include "pa_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int32_t x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

// Checks the cache description; fills `c`.
int check_cache(const pa_cache_desc* d, pa::CacheArgs* c) {
    if (!d) return fail(PA_ERR_INVALID_ARG, "cache descriptor is NULL");
    if (!d->kv_cache) return fail(PA_ERR_INVALID_ARG, "kv_cache is NULL");
    if (d->num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks must be > 0 (got %d)", d->num_blocks);
    if (d->num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads must be > 0 (got %d)", d->num_kv_heads);
    if (d->dtype != PA_F32 && d->dtype != PA_BF16 && d->dtype != PA_FP8_E4M3)
        return fail(PA_ERR_UNSUPPORTED, "dtype %d not supported", d->dtype);
    if (d->dtype == PA_FP8_E4M3 && !(d->kv_scale > 0.f && d->kv_scale <= 3.4e38f))
        return fail(PA_ERR_INVALID_ARG, "kv_scale must be finite and > 0 for an FP8 cache (got %g)", (double)d->kv_scale);
    if (d->head_size != 64 && d->head_size != 128)
        return fail(PA_ERR_UNSUPPORTED, "head_size %d not supported (64 or 128)", d->head_size);
    if (!is_pow2(d->block_size) || d->block_size > 256)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d must be a power of two <= 256", d->block_size);
    if ((int64_t)d->num_blocks * d->block_size >= (int64_t(1) << 31))
        return fail(PA_ERR_INVALID_ARG, "num_blocks * block_size must be < 2^31");
    if ((int64_t)d->num_kv_heads * d->head_size > (int64_t(1) << 20))
        return fail(PA_ERR_INVALID_ARG, "num_kv_heads * head_size too large");
    c->kv = d->kv_cache;
    c->num_blocks = d->num_blocks;
    c->block_size = d->block_size;
    c->block_shift = log2i(d->block_size);
    c->num_kv_heads = d->num_kv_heads;
    c->head_size = d->head_size;
    c->dtype = d->dtype;
    c->kv_scale = d->dtype == PA_FP8_E4M3 ? d->kv_scale : 1.f;
    c->kv_inv_scale = 1.f / c->kv_scale;
    c->plane_elems = (int64_t)d->num_blocks * d->block_size * d->num_kv_heads * d->head_size;
    return PA_OK;
}

int check_heads(const pa::CacheArgs& c, int32_t num_heads) {
    if (num_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_heads must be > 0 (got %d)", num_heads);
    if (num_heads % c.num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "num_heads %d is not a multiple of num_kv_heads %d", num_heads,
                    c.num_kv_heads);
    const int group = num_heads / c.num_kv_heads;
    if (c.dtype != PA_F32 && group > 16)
        return fail(PA_ERR_UNSUPPORTED, "bf16 decode supports up to 16 query heads per KV head (got %d)", group);
    if (c.dtype != PA_F32 && c.block_size < 16)
        return fail(PA_ERR_UNSUPPORTED, "bf16 and fp8 kernels need block_size >= 16 (got %d)", c.block_size);
    if (num_heads > 65535) return fail(PA_ERR_INVALID_ARG, "num_heads too large");
    return PA_OK;
}

int launch_status(hipError_t e) {
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
    g_last_error[0] = 0;
    return PA_OK;
}

// Chunks of the decode step list per group of 8 KV heads.  Automatic: as many as the
// device holds at once (every chunk then runs in one wave of workgroups and they finish
// together), each of at least 4 steps (128 keys) so short batches are not cut into pieces
// that cost more to merge than to stream.  partition_size > 0: chunks of at least that
// many keys, as many as a batch of max_seq_len sequences needs (tests use small ones to
// cut sequences many times).
struct Chunks {
    int32_t nw;
    int32_t min_steps;
};
Chunks decode_chunks(int32_t num_seqs, int32_t head_size, int32_t num_kv_heads, int32_t max_keys,
                     int32_t partition_size) {
    Chunks c;
    const int32_t ygroups = (num_kv_heads + 7) / 8;
    if (partition_size > 0) {
        c.min_steps = partition_size / 32;
        const int64_t smax = (int64_t)num_seqs * ((max_keys + 31) / 32);
        const int64_t nw = (smax + c.min_steps - 1) / c.min_steps;
        c.nw = (int32_t)(nw < 1 ? 1 : (nw > (1 << 24) ? (1 << 24) : nw));
    } else {
        c.min_steps = 4;
        const int64_t smax = (int64_t)num_seqs * ((max_keys + 31) / 32);
        const int64_t use = (smax + c.min_steps - 1) / c.min_steps;
        int32_t nw = pa::decode_resident_slots(head_size, num_kv_heads) / ygroups;
        if (nw > use) nw = (int32_t)use;
        c.nw = nw < 1 ? 1 : nw;
    }
    return c;
}

// Largest key span a sequence's steps cover: its live keys [lo, n) plus the < 32 keys
// between lo and the 32-aligned start of its first step.  start > 0: the keys after a
// shared prefix of that length.
int32_t max_keys_of(int32_t max_seq_len, int32_t window, int32_t start = 0) {
    if (start > 0) return max_seq_len > pa::decode_base(start) ? max_seq_len - pa::decode_base(start) : 0;
    if (window > 0 && max_seq_len > window) return max_seq_len < window + 31 ? max_seq_len : window + 31;
    return max_seq_len;
}

// The shared prefix's pass and its key chunks.  With many (sequence, query head) rows per KV
// head the pass runs on the prefill kernel (64-key tiles in LDS shared by four waves of 32
// rows), its chunks sized for about one workgroup per compute unit with at least two tiles
// each; with few rows that kernel has too few q-tiles to fill the device and the pass runs on
// the split-key kernel (16 rows per wave, the waves of a workgroup splitting the chunk's
// keys), with about one 8-wave workgroup per compute unit and at least two 32-key steps per
// wave.  Measured crossover: B 64 x G 4 = 256 rows favour the split-key kernel, 1024 rows the
// prefill kernel.
struct PrefixPlan {
    int32_t chunks;
    bool mfma;
};
PrefixPlan cascade_prefix_plan(int32_t num_seqs, int32_t group, int32_t num_kv_heads, int32_t P) {
    PrefixPlan p;
    p.mfma = (int64_t)num_seqs * group >= 512;
    int64_t nc, most;
    if (p.mfma) {
        const int64_t wpc = pa::prefix_workgroups_per_chunk(num_seqs, group, num_kv_heads);
        const int64_t tiles = pa::prefix_tiles(P);
        nc = (256 + wpc - 1) / wpc;
        most = tiles / 2;
    } else {
        const int64_t steps = (P + 31) / 32;
        const int64_t units = (((int64_t)num_seqs * group + 15) / 16) * num_kv_heads;
        nc = (256 + units - 1) / units;
        most = steps / 16;
    }
    if (nc > most) nc = most;
    if (nc > 64) nc = 64;
    p.chunks = (int32_t)(nc < 1 ? 1 : nc);
    return p;
}

// Workspace bytes of a decode launch: partial states of the chunk split (none with a
// single chunk or a float32 cache), then, with a shared prefix, the prefix chunks' states.
struct DecodePlan {
    Chunks c;
    int32_t prefix_chunks;
    bool prefix_mfma;
    size_t chunk_bytes;
    size_t prefix_bytes;
};
DecodePlan decode_plan(const pa_cache_desc* cache, int32_t num_seqs, int32_t num_heads, int32_t max_seq_len,
                       int32_t window, int32_t key_start, int32_t partition_size) {
    DecodePlan p = {{1, 1}, 0, false, 0, 0};
    if (cache->dtype == PA_F32) return p;
    p.c = decode_chunks(num_seqs, cache->head_size, cache->num_kv_heads,
                        max_keys_of(max_seq_len, window > 0 ? window : 0, key_start), partition_size);
    if (p.c.nw > 1) p.chunk_bytes = (size_t)p.c.nw * 2 * num_heads * ((size_t)cache->head_size + 2) * sizeof(float);
    if (key_start > 0) {
        const PrefixPlan pp = cascade_prefix_plan(num_seqs, num_heads / cache->num_kv_heads, cache->num_kv_heads, key_start);
        p.prefix_chunks = pp.chunks;
        p.prefix_mfma = pp.mfma;
        p.prefix_bytes = (size_t)p.prefix_chunks * num_seqs * num_heads * ((size_t)cache->head_size + 2) * sizeof(float);
    }
    return p;
}

// Scratch of pa_decode_no_alloc: one array on each GPU the library's code is loaded on.
// In host code its name is a host-side stand-in, not a device address; the address comes
// from hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) char scratch[PA_DECODE_NO_ALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device.  Concurrent first calls on one device
// may each look it up; they store the same address.
int scratch_address(void** ptr) {
    static std::atomic<void*> addr[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d out of range", dev);
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(PA_ERR_LAUNCH, "no device address for the decode scratch on device %d: %s", dev,
                        hipGetErrorString(e));
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PA_ERR_WORKSPACE: return "workspace too small";
        case PA_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

const char* pa_last_error(void) { return g_last_error; }

int pa_store_kv(const pa_cache_desc* cache, const void* key, const void* value,
                const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
    pa::StoreArgs a;
    int st = check_cache(cache, &a.c);
    if (st) return st;
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (num_tokens == 0) { g_last_error[0] = 0; return PA_OK; }
    if (!key || !value || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "key, value and slot_mapping must be non-NULL");
    a.key = key;
    a.value = value;
    a.slots = slot_mapping;
    a.num_tokens = num_tokens;
    return launch_status(pa::launch_store(a, (hipStream_t)stream));
}

int pa_copy_blocks(const pa_cache_desc* cache, const int32_t* block_pairs, int32_t num_pairs,
                   void* stream) {
    pa::CopyArgs a;
    int st = check_cache(cache, &a.c);
    if (st) return st;
    if (num_pairs < 0 || num_pairs > (1 << 29)) return fail(PA_ERR_INVALID_ARG, "num_pairs out of range (got %d)", num_pairs);
    if (num_pairs == 0) { g_last_error[0] = 0; return PA_OK; }
    if (!block_pairs) return fail(PA_ERR_INVALID_ARG, "block_pairs is NULL");
    a.pairs = block_pairs;
    a.num_pairs = num_pairs;
    return launch_status(pa::launch_copy_blocks(a, (hipStream_t)stream));
}

static int prefill_args(const pa_cache_desc* cache, void* out, const void* query,
                        const int32_t* block_table, int32_t max_blocks_per_seq,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                        int32_t num_heads, float scale, int32_t sliding_window, const float* alibi_slopes,
                        pa::PrefillArgs* pa_out, bool* empty) {
    pa::PrefillArgs& a = *pa_out;
    *empty = false;
    int st = check_cache(cache, &a.c);
    if (st) return st;
    if ((st = check_heads(a.c, num_heads))) return st;
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
    if (max_seqlen_q < 0 || max_seqlen_k < 0) return fail(PA_ERR_INVALID_ARG, "max_seqlen_q/k must be >= 0");
    if (num_seqs == 0 || max_seqlen_q == 0) { *empty = true; return PA_OK; }
    if (!out || !query || !block_table || !cu_seqlens_q || !cu_seqlens_k)
        return fail(PA_ERR_INVALID_ARG, "out, query, block_table, cu_seqlens_q and cu_seqlens_k must be non-NULL");
    if (max_blocks_per_seq < 1) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
    if ((int64_t)max_seqlen_k > (int64_t)max_blocks_per_seq * a.c.block_size)
        return fail(PA_ERR_INVALID_ARG, "max_seqlen_k %d exceeds max_blocks_per_seq * block_size", max_seqlen_k);
    // > 0 and finite: the kernels fold the scale into the exponent, where a masked score (-inf)
    // times a zero or infinite scale would give NaN instead of a zero weight
    if (!(scale > 0.f && scale <= 3.4e38f))
        return fail(PA_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
    if (a.c.dtype == PA_F32 && (int64_t)num_seqs * max_seqlen_q >= (int64_t(1) << 31))
        return fail(PA_ERR_INVALID_ARG, "num_seqs * max_seqlen_q too large");
    if ((int64_t)num_seqs * num_heads * ((max_seqlen_q + 31) / 32) >= (int64_t(1) << 30))
        return fail(PA_ERR_INVALID_ARG, "grid too large");
    a.out = out;
    a.q = query;
    a.table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.num_seqs = num_seqs;
    a.max_seqlen_q = max_seqlen_q;
    a.num_heads = num_heads;
    a.group = num_heads / a.c.num_kv_heads;
    a.scale = scale;
    a.window = sliding_window > 0 ? sliding_window : 0;
    a.knew = nullptr;
    a.vnew = nullptr;
    a.slots = nullptr;
    a.alibi = alibi_slopes;
    a.prefix_len = 0;
    a.prefix_chunks = 0;
    a.pre_o = nullptr;
    a.pre_ml = nullptr;
    a.cascade = 0;
    a.prefix_rows = 0;
    return PA_OK;
}

int pa_prefill_varlen(const pa_cache_desc* cache, void* out, const void* query,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                      int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                      int32_t num_heads, float scale, int32_t sliding_window,
                      const float* alibi_slopes, void* stream) {
    pa::PrefillArgs a;
    bool empty;
    int st = prefill_args(cache, out, query, block_table, max_blocks_per_seq, cu_seqlens_q, cu_seqlens_k,
                          num_seqs, max_seqlen_q, max_seqlen_k, num_heads, scale, sliding_window,
                          alibi_slopes, &a, &empty);
    if (st) return st;
    if (empty) { g_last_error[0] = 0; return PA_OK; }
    hipStream_t s = (hipStream_t)stream;
    return launch_status(a.c.dtype == PA_F32 ? pa::launch_prefill_f32(a, s) : pa::launch_prefill_bf16(a, s));
}

int pa_prefill_varlen_with_store(const pa_cache_desc* cache, void* out, const void* query,
                                 const void* key, const void* value, const int32_t* slot_mapping,
                                 int32_t num_tokens, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, int32_t num_heads, float scale,
                                 int32_t sliding_window, const float* alibi_slopes, void* stream) {
    pa::PrefillArgs a;
    bool empty;
    int st = prefill_args(cache, out, query, block_table, max_blocks_per_seq, cu_seqlens_q, cu_seqlens_k,
                          num_seqs, max_seqlen_q, max_seqlen_k, num_heads, scale, sliding_window,
                          alibi_slopes, &a, &empty);
    if (st) return st;
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (num_tokens > 0 && (!key || !value || !slot_mapping))
        return fail(PA_ERR_INVALID_ARG, "key, value and slot_mapping must be non-NULL");
    if (empty || num_tokens == 0) {
        if (num_tokens == 0 && !empty)
            return fail(PA_ERR_INVALID_ARG, "num_tokens is 0 but the batch has query rows");
        g_last_error[0] = 0;
        return PA_OK;
    }
    hipStream_t s = (hipStream_t)stream;
    if (a.c.dtype == PA_BF16) {
        a.knew = key;
        a.vnew = value;
        a.slots = slot_mapping;
        return launch_status(pa::launch_prefill_bf16(a, s));
    }
    // float32 and FP8 caches: the store, then the attention, on the same stream (an FP8 cache
    // must hold the quantized new rows before the attention reads them)
    pa::StoreArgs sa;
    sa.c = a.c;
    sa.key = key;
    sa.value = value;
    sa.slots = slot_mapping;
    sa.num_tokens = num_tokens;
    hipError_t e = pa::launch_store(sa, s);
    if (e != hipSuccess) return launch_status(e);
    return launch_status(a.c.dtype == PA_F32 ? pa::launch_prefill_f32(a, s) : pa::launch_prefill_bf16(a, s));
}

size_t pa_decode_workspace_size(const pa_cache_desc* cache, int32_t num_seqs, int32_t num_heads,
                                int32_t max_seq_len, int32_t sliding_window, int32_t partition_size) {
    if (!cache || num_seqs <= 0 || num_heads <= 0 || max_seq_len <= 0 || partition_size < 0) return 0;
    if (cache->num_kv_heads <= 0 || num_heads % cache->num_kv_heads != 0) return 0;
    return decode_plan(cache, num_seqs, num_heads, max_seq_len, sliding_window, 0, partition_size).chunk_bytes;
}

size_t pa_cascade_decode_workspace_size(const pa_cache_desc* cache, int32_t num_seqs, int32_t num_heads,
                                        int32_t max_seq_len, int32_t common_prefix_len,
                                        int32_t partition_size) {
    if (!cache || num_seqs <= 0 || num_heads <= 0 || max_seq_len <= 0 || partition_size < 0) return 0;
    if (cache->num_kv_heads <= 0 || num_heads % cache->num_kv_heads != 0 || common_prefix_len < 0) return 0;
    const DecodePlan p = decode_plan(cache, num_seqs, num_heads, max_seq_len, 0, common_prefix_len, partition_size);
    return p.chunk_bytes + p.prefix_bytes;
}

// Validation and launch planning shared by pa_decode and pa_decode_with_store; *empty is
// set when there is nothing to launch.
static int decode_args(const pa_cache_desc* cache, void* out, const void* query, const int32_t* block_table,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                       int32_t max_seq_len, int32_t num_heads, float scale, int32_t sliding_window,
                       const float* alibi_slopes, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, pa::DecodeArgs* a_out, bool* empty, int32_t key_start = 0) {
    pa::DecodeArgs& a = *a_out;
    *empty = false;
    int st = check_cache(cache, &a.c);
    if (st) return st;
    if ((st = check_heads(a.c, num_heads))) return st;
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
    if (max_seq_len < 0) return fail(PA_ERR_INVALID_ARG, "max_seq_len must be >= 0");
    if (num_seqs == 0) { *empty = true; return PA_OK; }
    if (!out || !query || !block_table || !seq_lens)
        return fail(PA_ERR_INVALID_ARG, "out, query, block_table and seq_lens must be non-NULL");
    if (max_blocks_per_seq < 1) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
    if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * a.c.block_size)
        return fail(PA_ERR_INVALID_ARG, "max_seq_len %d exceeds max_blocks_per_seq * block_size", max_seq_len);
    if (partition_size < 0 || partition_size % 32 != 0)
        return fail(PA_ERR_INVALID_ARG, "partition_size must be 0 or a positive multiple of 32 (got %d)", partition_size);
    // > 0 and finite: the kernels fold the scale into the exponent, where a masked score (-inf)
    // times a zero or infinite scale would give NaN instead of a zero weight
    if (!(scale > 0.f && scale <= 3.4e38f))
        return fail(PA_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
    const int32_t win = sliding_window > 0 ? sliding_window : 0;
    if ((int64_t)num_seqs * ((max_keys_of(max_seq_len, win, key_start) + 31) / 32 + 1) > 0x7fffffff)
        return fail(PA_ERR_INVALID_ARG, "num_seqs * max_seq_len too large");
    a.out = out;
    a.q = query;
    a.table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.seq_lens = seq_lens;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.group = num_heads / a.c.num_kv_heads;
    a.scale = scale;
    a.window = win;
    a.alibi = alibi_slopes;
    a.nw = 1;
    a.min_steps = 1;
    a.ws_o = nullptr;
    a.ws_ml = nullptr;
    a.key_start = key_start;
    a.knew = nullptr;
    a.vnew = nullptr;
    a.slots = nullptr;
    a.prefix_chunks = 0;
    a.prefix_mfma = 0;
    a.pre_o = nullptr;
    a.pre_ml = nullptr;
    if (a.c.dtype == PA_F32) return PA_OK;
    if (a.c.num_kv_heads > 65535) return fail(PA_ERR_INVALID_ARG, "num_kv_heads too large");
    const DecodePlan p = decode_plan(cache, num_seqs, num_heads, max_seq_len, win, key_start, partition_size);
    const size_t need = p.chunk_bytes + p.prefix_bytes;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PA_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need, workspace ? workspace_bytes : 0);
    if (need > 0 && ((uintptr_t)workspace & 15) != 0)
        return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (p.chunk_bytes > 0) {
        a.nw = p.c.nw;
        a.min_steps = p.c.min_steps;
        a.ws_o = (float*)workspace;
        a.ws_ml = a.ws_o + (size_t)p.c.nw * 2 * num_heads * a.c.head_size;
    }
    if (p.prefix_bytes > 0) {
        a.prefix_chunks = p.prefix_chunks;
        a.prefix_mfma = p.prefix_mfma ? 1 : 0;
        a.pre_o = (float*)((char*)workspace + p.chunk_bytes);
        a.pre_ml = a.pre_o + (size_t)p.prefix_chunks * num_seqs * num_heads * a.c.head_size;
    }
    return PA_OK;
}

int pa_decode(const pa_cache_desc* cache, void* out, const void* query, const int32_t* block_table,
              int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
              int32_t max_seq_len, int32_t num_heads, float scale, int32_t sliding_window,
              const float* alibi_slopes, int32_t partition_size, void* workspace,
              size_t workspace_bytes, void* stream) {
    pa::DecodeArgs a;
    bool empty;
    int st = decode_args(cache, out, query, block_table, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len,
                         num_heads, scale, sliding_window, alibi_slopes, partition_size, workspace,
                         workspace_bytes, &a, &empty);
    if (st) return st;
    if (empty) { g_last_error[0] = 0; return PA_OK; }
    hipStream_t s = (hipStream_t)stream;
    return launch_status(a.c.dtype == PA_F32 ? pa::launch_decode_f32(a, s) : pa::launch_decode_bf16(a, s));
}

int pa_decode_no_alloc(const pa_cache_desc* cache, void* out, const void* query, const int32_t* block_table,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                       int32_t max_seq_len, int32_t num_heads, float scale, int32_t sliding_window,
                       const float* alibi_slopes, int32_t partition_size, void* stream) {
    pa::DecodeArgs a;
    bool empty;
    // the split's size first (0 for invalid arguments, which decode_args then rejects)
    const size_t need = pa_decode_workspace_size(cache, num_seqs, num_heads, max_seq_len, sliding_window,
                                                 partition_size);
    if (need > PA_DECODE_NO_ALLOC_SCRATCH_BYTES) {
        // any other invalid argument is reported first, as pa_decode would
        const int st = decode_args(cache, out, query, block_table, max_blocks_per_seq, seq_lens, num_seqs,
                                   max_seq_len, num_heads, scale, sliding_window, alibi_slopes, partition_size,
                                   nullptr, 0, &a, &empty);
        if (st != PA_OK && st != PA_ERR_WORKSPACE) return st;
        return fail(PA_ERR_WORKSPACE,
                    "pa_decode_no_alloc: this split needs %zu bytes of scratch, more than its maximum of %u "
                    "(pa_decode with a workspace serves it)", need, (unsigned)PA_DECODE_NO_ALLOC_SCRATCH_BYTES);
    }
    void* ws = nullptr;
    if (need > 0) {
        const int st = scratch_address(&ws);
        if (st) return st;
    }
    int st = decode_args(cache, out, query, block_table, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len,
                         num_heads, scale, sliding_window, alibi_slopes, partition_size, ws,
                         need > 0 ? (size_t)PA_DECODE_NO_ALLOC_SCRATCH_BYTES : 0, &a, &empty);
    if (st) return st;
    if (empty) { g_last_error[0] = 0; return PA_OK; }
    hipStream_t s = (hipStream_t)stream;
    return launch_status(a.c.dtype == PA_F32 ? pa::launch_decode_f32(a, s) : pa::launch_decode_bf16(a, s));
}

int pa_decode_with_store(const pa_cache_desc* cache, void* out, const void* query, const void* key,
                         const void* value, const int32_t* slot_mapping, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t max_seq_len, int32_t num_heads, float scale, int32_t sliding_window,
                         const float* alibi_slopes, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, void* stream) {
    pa::DecodeArgs a;
    bool empty;
    int st = decode_args(cache, out, query, block_table, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len,
                         num_heads, scale, sliding_window, alibi_slopes, partition_size, workspace,
                         workspace_bytes, &a, &empty);
    if (st) return st;
    if (empty) { g_last_error[0] = 0; return PA_OK; }
    if (!key || !value || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "key, value and slot_mapping must be non-NULL");
    hipStream_t s = (hipStream_t)stream;
    if (a.c.dtype == PA_BF16) {  // one launch: the decode kernel reads and stores the new rows
        a.knew = key;
        a.vnew = value;
        a.slots = slot_mapping;
        return launch_status(pa::launch_decode_bf16(a, s));
    }
    pa::StoreArgs sa;
    sa.c = a.c;
    sa.key = key;
    sa.value = value;
    sa.slots = slot_mapping;
    sa.num_tokens = num_seqs;
    hipError_t e = pa::launch_store(sa, s);
    if (e != hipSuccess) return launch_status(e);
    return launch_status(a.c.dtype == PA_F32 ? pa::launch_decode_f32(a, s) : pa::launch_decode_bf16(a, s));
}

size_t pa_cascade_prefill_varlen_workspace_size(const pa_cache_desc* cache, int32_t num_tokens, int32_t num_heads,
                                                int32_t common_prefix_len) {
    if (!cache || num_tokens <= 0 || num_heads <= 0 || common_prefix_len <= 0) return 0;
    if (cache->num_kv_heads <= 0 || num_heads % cache->num_kv_heads != 0 || cache->dtype == PA_F32) return 0;
    const PrefixPlan pp = cascade_prefix_plan(num_tokens, num_heads / cache->num_kv_heads, cache->num_kv_heads,
                                              common_prefix_len);
    return (size_t)pp.chunks * num_tokens * num_heads * ((size_t)cache->head_size + 2) * sizeof(float);
}

int pa_cascade_prefill_varlen(const pa_cache_desc* cache, void* out, const void* query,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads, float scale,
                              int32_t common_prefix_len, int32_t num_tokens, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (cache && cache->dtype == PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "shared-prefix prefill needs a bf16 or FP8 cache");
    if (cache && (cache->block_size <= 0 || common_prefix_len < 0 || common_prefix_len % cache->block_size != 0))
        return fail(PA_ERR_INVALID_ARG, "common_prefix_len must be a non-negative multiple of block_size (got %d)",
                    common_prefix_len);
    pa::PrefillArgs a;
    bool empty;
    int st = prefill_args(cache, out, query, block_table, max_blocks_per_seq, cu_seqlens_q, cu_seqlens_k,
                          num_seqs, max_seqlen_q, max_seqlen_k, num_heads, scale, 0, nullptr, &a, &empty);
    if (st) return st;
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (empty || num_tokens == 0) {
        if (num_tokens == 0 && !empty) return fail(PA_ERR_INVALID_ARG, "num_tokens is 0 but the batch has query rows");
        g_last_error[0] = 0;
        return PA_OK;
    }
    if (common_prefix_len > max_seqlen_k)
        return fail(PA_ERR_INVALID_ARG, "common_prefix_len %d exceeds max_seqlen_k %d", common_prefix_len, max_seqlen_k);
    hipStream_t s = (hipStream_t)stream;
    if (common_prefix_len == 0) return launch_status(pa::launch_prefill_bf16(a, s));
    const PrefixPlan pp = cascade_prefix_plan(num_tokens, a.group, a.c.num_kv_heads, common_prefix_len);
    const size_t need = (size_t)pp.chunks * num_tokens * num_heads * ((size_t)a.c.head_size + 2) * sizeof(float);
    if (!workspace || workspace_bytes < need)
        return fail(PA_ERR_WORKSPACE, "shared-prefix prefill needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : 0);
    if (((uintptr_t)workspace & 15) != 0) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if ((int64_t)8 * (((int64_t)num_tokens * a.group + 15) / 16) * (((int64_t)a.c.num_kv_heads * pp.chunks + 7) / 8) >
        0x7fffffff)
        return fail(PA_ERR_INVALID_ARG, "num_tokens * num_heads too large for the prefix pass");
    // the prefix pass: every packed query row against the shared prefix, read through table row 0
    pa::DecodeArgs d;
    memset(&d, 0, sizeof(d));
    d.c = a.c;
    d.q = query;
    d.table = block_table;
    d.max_blocks = max_blocks_per_seq;
    d.num_seqs = num_tokens;
    d.num_heads = num_heads;
    d.group = a.group;
    d.scale = scale;
    d.key_start = common_prefix_len;
    d.prefix_chunks = pp.chunks;
    d.prefix_mfma = pp.mfma ? 1 : 0;
    d.pre_o = (float*)workspace;
    d.pre_ml = d.pre_o + (size_t)pp.chunks * num_tokens * num_heads * a.c.head_size;
    hipError_t e = pa::launch_prefix_pass(d, s);
    if (e != hipSuccess) return launch_status(e);
    // each sequence's own keys, folding the prefix states in
    a.cascade = 1;
    a.prefix_len = common_prefix_len;
    a.prefix_chunks = pp.chunks;
    a.prefix_rows = num_tokens;
    a.pre_o = d.pre_o;
    a.pre_ml = d.pre_ml;
    return launch_status(pa::launch_prefill_bf16(a, s));
}

int pa_cascade_decode(const pa_cache_desc* cache, void* out, const void* query, const int32_t* block_table,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                      int32_t max_seq_len, int32_t num_heads, float scale, int32_t common_prefix_len,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
    if (cache && cache->dtype == PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "shared-prefix decode needs a bf16 cache");
    if (cache && (cache->block_size <= 0 || common_prefix_len < 0 || common_prefix_len % cache->block_size != 0))
        return fail(PA_ERR_INVALID_ARG, "common_prefix_len must be a non-negative multiple of block_size (got %d)",
                    common_prefix_len);
    if (num_seqs > 0 && common_prefix_len > max_seq_len)
        return fail(PA_ERR_INVALID_ARG, "common_prefix_len %d exceeds max_seq_len %d", common_prefix_len, max_seq_len);
    pa::DecodeArgs a;
    bool empty;
    int st = decode_args(cache, out, query, block_table, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len,
                         num_heads, scale, 0, nullptr, partition_size, workspace, workspace_bytes, &a, &empty,
                         common_prefix_len);
    if (st) return st;
    if (empty) { g_last_error[0] = 0; return PA_OK; }
    if ((int64_t)8 * (((int64_t)num_seqs * a.group + 15) / 16) * (((int64_t)a.c.num_kv_heads * a.prefix_chunks + 7) / 8) >
        0x7fffffff)
        return fail(PA_ERR_INVALID_ARG, "num_seqs * num_heads too large for the prefix pass");
    hipStream_t s = (hipStream_t)stream;
    if (common_prefix_len == 0) return launch_status(pa::launch_decode_bf16(a, s));
    return launch_status(pa::launch_cascade_decode_bf16(a, s));
}

}  // extern "C"
