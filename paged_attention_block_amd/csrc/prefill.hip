// Varlen causal paged prefill for bf16 and FP8 caches on gfx950 (MFMA, fp32 online softmax).
//
// The operation (MinivLLM API docs, "Attention", flash_attention_prefill; HF transformers
// continuous_batching input_ouputs.py, build_attention_mask): packed query chunks, causal
// diagonal offset by seqlen_k - seqlen_q, optional sliding window of W keys ending at the
// query's own position, GQA, keys read through the block table (vLLM learning book
// section 5).
//
// Work item = one 4-wave workgroup per (sequence, KV head, q-tile, part of the tile's
// (query head, 32-row block) pairs).  Wave w owns one query head of the KV head's group and
// 32 rows; all waves share the K/V tiles (64 keys) staged in LDS, so a K/V byte is fetched
// once per workgroup for up to four heads.  Per 64-key tile each wave computes
//   S^T[64 keys x 32 rows] = K . Q^T      (bf16 MFMA, K from LDS, Q^T in VGPRs)
//   online softmax on S^T, P^T packed to bf16 straight from the accumulators
//   O^T[D x 32 rows]   += V^T . P^T        (V^T from LDS)
// in one of two MFMA forms (kPrefillW32 picks): 32x32x16, where lane l owns query row l % 32
// and half of its keys (16 MFMAs per product; the row's maximum and sum combine lanes l and
// l ^ 32 only), or 16x16x32 (32 MFMAs per product, two 16-row blocks per wave).
// K and V rows go from HBM straight into LDS (global_load_lds, 16 B per lane, no register
// staging), two tiles deep, so the copy of tile i+1 overlaps the math of tile i.  The
// V^T operand is read with the transposing LDS read (ds_read_b64_tr_b16): within a
// 16-lane group, lane i receives element i%4 of the 4-element vectors addressed by lanes
// i/4 + 4j, so when source lane s addresses row base + s/4, dims d0 + 4*(s%4), lane i
// receives 4 consecutive keys at dim d0 + i -- the MFMA layout, from a row-major tile.
// LDS rows are packed; the 16-byte chunks of row r are XOR-swizzled (K: chunk ^ (r & 15),
// V: chunk ^ 4*(r & 3)) so the operand reads hit distinct banks.  The swizzle is applied
// on the global side: a lane fetches the global chunk that belongs at its fixed LDS slot.
//
// Tiles outside the union of the rows' live key ranges are never visited; inside a
// visited tile, keys outside that union are copied from a live block of the same tile
// (never through an unread block-table entry) and then overwritten with zeros in LDS by
// the wave that copied them, so cache slots outside every row's window may hold anything.
// Tiles crossing the causal diagonal or the window edge get an element mask.
// The bf16 output of a wave (32 rows x D) goes through an LDS buffer no wave reads any more,
// so that each global store writes whole 256-byte rows rather than 8-byte pieces of 32 rows.
//
// Workgroups are numbered so that each XCD (work dispatched round-robin over 8) runs the
// q-tiles of one (sequence, KV head) back to back: those share K/V through that XCD's L2.
#include <math.h>

#include <type_traits>

#include "pa_internal.hpp"

namespace pa {

// Tile copies and their waits are inline assembly.  A copy's rows are visible to the other
// waves of the workgroup only once the copying wave has waited for its copies and the
// workgroup has then passed a barrier, so each wave waits for its own copies (wait_vmcnt)
// right before the barrier: a wait the compiler places itself comes at the first read of the
// tile, after the barrier.  Copies the compiler cannot see never make its own waits unsafe
// (vmcnt counts complete in order; extra outstanding operations only make a wait stricter).
// The compiler's LDS-copy builtin, which it tracks per LDS buffer, measured no faster issued
// where these copies are; spread between the S^T MFMAs it cost the copies lead time, which
// the workloads whose K/V comes from HBM need (the mixed step 6% slower).

// one 16-byte-per-lane copy HBM -> LDS: lane l's 16 bytes at base + voff (base wave-uniform,
// voff the lane's 32-bit offset) land at LDS byte address lds + 16*l (lds wave-uniform)
__device__ __forceinline__ void copy_to_lds16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// Four (two) such copies under one M0 write: copy j takes lane offset voff[j] and lands at LDS
// byte lds + S*j + 16*l.  The instruction's immediate offset is added to both the global and
// the LDS address, so copy j carries S*j there and voff[j] is the lane's offset less S*j.
template <int S>
__device__ __forceinline__ void copy4_to_lds16(const void* base, const uint32_t (&voff)[4], uint32_t lds) {
    static_assert(3 * S < 4096, "immediate offsets are 12 bits");
    asm volatile("s_mov_b32 m0, %5\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %4\n\t"
                 "global_load_lds_dwordx4 %1, %4 offset:%6\n\t"
                 "global_load_lds_dwordx4 %2, %4 offset:%7\n\t"
                 "global_load_lds_dwordx4 %3, %4 offset:%8"
                 :
                 : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(base), "s"(lds), "i"(S), "i"(2 * S),
                   "i"(3 * S)
                 : "memory", "m0");
}
template <int S>
__device__ __forceinline__ void copy2_to_lds16(const void* base, const uint32_t (&voff)[2], uint32_t lds) {
    static_assert(S < 4096, "immediate offsets are 12 bits");
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %2\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:%4"
                 :
                 : "v"(voff[0]), "v"(voff[1]), "s"(base), "s"(lds), "i"(S)
                 : "memory", "m0");
}

// the same copy from a per-lane 64-bit address
__device__ __forceinline__ void copy_to_lds16_lane(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(n) for a wave-uniform n (the count is an instruction immediate; counts
// above 23 wait for everything, which is always safe)
__device__ __forceinline__ void wait_vmcnt(int n) {
#define PA_VMCNT_CASE(N) \
    case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
    switch (n) {
        PA_VMCNT_CASE(1) PA_VMCNT_CASE(2) PA_VMCNT_CASE(3) PA_VMCNT_CASE(4) PA_VMCNT_CASE(5)
        PA_VMCNT_CASE(6) PA_VMCNT_CASE(7) PA_VMCNT_CASE(8) PA_VMCNT_CASE(9) PA_VMCNT_CASE(10)
        PA_VMCNT_CASE(11) PA_VMCNT_CASE(12) PA_VMCNT_CASE(13) PA_VMCNT_CASE(14) PA_VMCNT_CASE(15)
        PA_VMCNT_CASE(16) PA_VMCNT_CASE(17) PA_VMCNT_CASE(18) PA_VMCNT_CASE(19) PA_VMCNT_CASE(20)
        PA_VMCNT_CASE(21) PA_VMCNT_CASE(22) PA_VMCNT_CASE(23)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
#undef PA_VMCNT_CASE
}

// workgroup barrier after this wave's LDS writes completed; no wait for copies in flight
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// the same barrier, holding `ready` (a scalar load issued before it) as an input, so that the
// load is issued ahead of the barrier and its latency runs under the barrier's wait
__device__ __forceinline__ void lds_barrier_after(int ready) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::"s"(ready) : "memory");
}

// Waves per workgroup (W): the workgroup's waves share each K/V tile staged in LDS.  Four
// waves, two workgroups per CU, measured faster than one 8-wave workgroup per CU sharing
// every tile (whose waves run the same stage at the same time on a SIMD).
constexpr int kPrefillWaves = 4;
// Waves each SIMD holds at once (the register budget: 512 / this many VGPRs per wave).
constexpr int kPrefillWavesPerSimd = 2;
// Keys per compute step of the 32x32x16 form: a K/V tile is processed in steps of this many
// keys (S^T, softmax and P.V of one step before the next), which bounds the live S registers.
constexpr int kPrefillCB = 64;

// Work decomposition.  A q-tile is rb blocks of 32 query rows of one (sequence, KV head);
// its (query head of the group, row block) pairs, row block major, are dealt W at a time to
// W-wave workgroups (rb = W / gcd(G, W), so the G * rb pairs fill whole workgroups for every
// group size G and no wave idles).
struct PrefillGrid {
    int rb;             // 32-row blocks per q-tile
    int wgs_per_tile;   // G * rb / W
    int n_sg;           // num_seqs * num_kv_heads
    int n_tiles;        // ceil(max_seqlen_q / (32 * rb)) * wgs_per_tile
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// max / sum of lanes l and l ^ 32 (the two halves of a query row's keys in the 32x32 form)
__device__ inline float half_max(float v) {
    const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}
__device__ inline float half_sum(float v) {
    const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false, false);
    return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
}

// two E4M3 codes (bytes 0-1, or 2-3 with hi) -> two bf16, exactly
__device__ inline uint32_t e4m3x2_to_bf16(uint32_t w, bool hi) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false));
}
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// FP8: the cache holds E4M3 codes of K / kv_scale and V / kv_scale.  A tile copy is then a
// register-staged 8-byte load per lane, widened exactly to bf16 (every E4M3 value is a bf16
// value) and written to the same swizzled LDS slot the bf16 copy fills, so the MFMA operand
// reads are unchanged; kv_scale joins the softmax scale and the output normalisation.
//
// PREFIX: the shared-prefix pass of cascade decode.  The "sequence" is the batch's decode
// queries (query[B][H][D] is a packed query block of B rows), the keys are chunk c of the
// shared prefix [0, prefix_len) read through table row 0, every query sees every key of the
// chunk (no causal diagonal; the chunk's last partial tile is masked at its end), and each
// (chunk, row, head) leaves its unnormalised state (O, m, l) in pre_o / pre_ml instead of a
// bf16 output row.  Work item numbering treats (chunk, KV head) as the (sequence, KV head)
// index, so the q-tiles of one chunk and KV head share its K/V through one XCD's L2.
//
// CASC: the own-keys pass of shared-prefix prefill.  Each sequence attends only its keys from
// prefix_len on (keys below it are masked like a window's), and the epilogue folds in, by
// log-sum-exp, the states the prefix pass left for the same packed query row and head.
template <int D, int NBR, int BN, int NBUF, bool ALIBI, bool FP8, bool PREFIX, bool W32, bool CASC, bool FUSED>
__global__ __launch_bounds__(64 * kPrefillWaves, kPrefillWavesPerSimd) void prefill_bf16_kernel(const PrefillArgs a,
                                                                                                 const PrefillGrid pg) {
    constexpr int NGA = BN / 16;      // 16-key groups per K/V tile
    constexpr int NCC = BN / 32;      // 32-key chunks per K/V tile (PV MFMA k-steps)
    constexpr int RPW = 16 * NBR;     // query rows per wave (NBR blocks of 16)
    static_assert(RPW == 32, "row blocks of 32");
    constexpr int KS = D / 32;        // k-slices of q.K^T
    constexpr int DB = D / 16;        // 16-dim output blocks
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;     // rows per 1 KB copy instruction
    constexpr int NQ = BN / RPI;      // copy instructions per plane per tile
    constexpr int TILE = BN * D * 2;  // bytes of one plane of one tile
    constexpr int KSW = CPR >= 16 ? 15 : CPR - 1;        // K swizzle mask
    // V swizzle: chunk c of row r sits at slot c ^ vswz(r).  The transposing V^T reads of
    // lanes 0-31 cover rows r0..r0+3 and four consecutive chunks; XOR with 4 * (r & 3) puts the
    // 16 (row, chunk) pairs on distinct slots of a 256-byte row span, which keeps these 8-byte
    // reads free of LDS bank conflicts (counter: 0; the earlier 2 * (r & 7) pattern had two-way
    // conflicts on a third of the LDS-active cycles)
    auto vswz = [](int r) { return (4 * (r & 3)) & (CPR - 1); };
    constexpr int ELT = FP8 ? 1 : 2;  // bytes per cache element
    static_assert(!FP8 || NBUF == 2, "the FP8 copy stages one tile in registers");
    static_assert(!W32 || BN == 64 || BN == 32, "the 32x32x16 form takes tiles of one or two 32-key blocks");
    constexpr int CB = BN < kPrefillCB ? BN : kPrefillCB;  // keys per compute step (32x32x16 form)
    static_assert(CB % 32 == 0 && BN % CB == 0, "compute steps of whole 32-key blocks");
    constexpr int NB32 = CB / 32;     // 32-key blocks per compute step
    static_assert(!CASC || (W32 && !PREFIX), "the shared-prefix own-keys pass uses the 32x32x16 form");

    // NBUF K and NBUF V buffers as distinct objects, so the compiler can tell a copy into one
    // from a read of another and does not wait for in-flight copies before every LDS read
    __shared__ __attribute__((aligned(1024))) char lds_k0[TILE];
    __shared__ __attribute__((aligned(1024))) char lds_k1[TILE];
    __shared__ __attribute__((aligned(1024))) char lds_k2[NBUF > 2 ? TILE : 16];
    __shared__ __attribute__((aligned(1024))) char lds_k3[NBUF > 3 ? TILE : 16];
    __shared__ __attribute__((aligned(1024))) char lds_v0[TILE];
    __shared__ __attribute__((aligned(1024))) char lds_v1[TILE];
    __shared__ __attribute__((aligned(1024))) char lds_v2[NBUF > 2 ? TILE : 16];
    __shared__ __attribute__((aligned(1024))) char lds_v3[NBUF > 3 ? TILE : 16];

    // ---------------------------------------------------------------- work item
    // Workgroups are numbered so that each XCD (work dispatched round-robin over 8) runs the
    // tiles of one (sequence, KV head) back to back, longest q-tiles first.
    const int b = blockIdx.x;
    const int xcd = b & 7;
    const int li = b >> 3;
    const int sg = (li / pg.n_tiles) * 8 + xcd;
    if (sg >= pg.n_sg) return;
    const int ti = pg.n_tiles - 1 - li % pg.n_tiles;
    const int qt = ti / pg.wgs_per_tile;
    const int jw = ti % pg.wgs_per_tile;
    const int s = PREFIX ? 0 : sg / a.c.num_kv_heads;
    const int g = sg % a.c.num_kv_heads;
    const int pc = PREFIX ? sg / a.c.num_kv_heads : 0;  // prefix chunk
    const int G = a.group;

    const int q0 = PREFIX ? 0 : a.cu_q[s];
    const int sq = PREFIX ? a.num_seqs : a.cu_q[s + 1] - q0;
    const int i0 = qt * 32 * pg.rb;
    // the rows of this workgroup's pairs: row blocks (W jw) / G .. (W jw + W - 1) / G
    const int wg_row0 = i0 + 32 * ((kPrefillWaves * jw) / G);
    if (wg_row0 >= sq) return;
    const int wg_row_end = min(i0 + 32 * ((kPrefillWaves * jw + kPrefillWaves - 1) / G + 1), sq);
    // PREFIX: chunk pc of the prefix = 64-key tiles [tb, te), keys [kc0, kc1)
    int kc0 = 0, kc1 = 0;
    if constexpr (PREFIX) {
        const int pt = (a.prefix_len + BN - 1) / BN;
        kc0 = BN * (int)((int64_t)pc * pt / a.prefix_chunks);
        kc1 = min(a.prefix_len, BN * (int)((int64_t)(pc + 1) * pt / a.prefix_chunks));
    }
    const int sk = PREFIX ? kc1 : a.cu_k[s + 1] - a.cu_k[s];
    const int off = sk - sq;
    const int W = PREFIX ? 0 : a.window;
    const int rows_end = sq;
    // first key this pass attends (CASC: the keys after the shared prefix); has_lo: keys below
    // a row's first key exist in visited tiles and take an element mask
    const int kstart = CASC ? a.prefix_len : 0;
    const bool has_lo = W > 0 || kstart > 0;

    const int tid = threadIdx.x;
    constexpr int nwaves = kPrefillWaves;  // the launch is always 64 * kPrefillWaves threads
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: copy setup stays scalar
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int pair = kPrefillWaves * jw + wave;  // (head, row block) pair of this wave
    const int hig = pair % G;              // head within the group
    const bool wave_ok = pair < G * pg.rb;
    const int h = g * G + hig;
    const int H = a.num_heads;
    const int Hkv = a.c.num_kv_heads;

    // key range of the whole workgroup (union over its rows)
    const int wg_lo = PREFIX ? kc0 : max(kstart, W > 0 ? max(0, off + wg_row0 - W + 1) : 0);
    const int wg_hi = PREFIX ? kc1 - 1 : min(off + wg_row_end - 1, sk - 1);
    // this wave's rows and key range
    const int r0 = i0 + RPW * (pair / G);
    const int r_last = min(r0 + RPW - 1, rows_end - 1);
    const bool wave_active = wave_ok && r0 < rows_end;
    // (PREFIX: every row sees keys [kc0, kc1); the mask then only cuts at kc1)
    const int wv_hi = PREFIX ? kc1 - 1 : min(off + r_last, sk - 1);
    const int wv_lo = PREFIX ? kc0 : max(kstart, W > 0 ? max(0, off + r0 - W + 1) : 0);
    const int wv_lo_max = PREFIX ? kc0 : max(kstart, W > 0 ? max(0, off + r_last - W + 1) : 0);
    const int wv_p_min = PREFIX ? kc1 - 1 : off + r0;

    const float c_log2 = a.scale * (FP8 ? a.c.kv_scale : 1.f) * 1.4426950408889634f;
    // ALiBi slope of this wave's head in log2 units (the bias slope * (j - p) is added to the
    // scaled score before the softmax)
    const float sl2 = ALIBI && wave_ok ? a.alibi[h] * 1.4426950408889634f : 0.f;
    // the same slope in raw-score units (the scale is > 0): the 32x32x16 form seeds the S^T
    // accumulators with the bias, so the softmax needs no separate bias pass
    const float sl2r = ALIBI ? sl2 / c_log2 : 0.f;
    const int BS = a.c.block_size;
    const int shift = a.c.block_shift;
    const char* __restrict__ kplane = (const char*)a.c.kv;
    const int64_t vdelta = a.c.plane_elems * ELT;
    // the block table through the constant address space: it is never written while the
    // kernel runs, so the (wave-uniform) lookups become scalar loads that do not share the
    // vector-memory counter with the in-flight tile copies
    typedef __attribute__((address_space(4))) const int32_t cint32;
    cint32* table = (cint32*)(a.table + (int64_t)s * a.max_blocks);
    const int64_t RB = (int64_t)Hkv * D * ELT;  // cache token-row bytes

    // ---------------------------------------------------------------- Q^T operands
    bf16x8 qf[NBR][KS];
    int prow[NBR], plo[NBR];
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb) {
        const int row = r0 + 16 * nb + col;
        const bool ok = wave_active && row < rows_end;
        const u32x4* src = (const u32x4*)((const __bf16*)a.q + ((int64_t)(q0 + (ok ? row : 0)) * H + (wave_ok ? h : 0)) * D);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const u32x4 x = src[4 * t + grp];
            qf[nb][t] = __builtin_bit_cast(bf16x8, ok ? x : (u32x4)(0u));
        }
        prow[nb] = PREFIX ? kc1 - 1 : off + row;
        plo[nb] = max(kstart, W > 0 ? max(0, off + row - W + 1) : 0);
    }

    // 32x32x16 form (W32): lane l owns query row r0 + l % 32 of the wave's 32 rows; its operand
    // k-slices are dims 16t + 8 * (l / 32) .. + 7, and its accumulators hold that row's scores
    // (keys 8 * (i / 4) + 4 * (l / 32) + i % 4 of a 32-key block) and output dims.
    const int lrow = lane & 31;
    const int lh = lane >> 5;
    bf16x8 qw[D / 16];
    f32x16 ow[D / 32];
    int prw = 0, plw = 0;
    float mw = -INFINITY, lw = 0.f;
    if constexpr (W32) {
        const int row = r0 + lrow;
        const bool ok = wave_active && row < rows_end;
        const u32x4* src = (const u32x4*)((const __bf16*)a.q + ((int64_t)(q0 + (ok ? row : 0)) * H + (wave_ok ? h : 0)) * D);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            const u32x4 x = src[2 * t + lh];
            qw[t] = __builtin_bit_cast(bf16x8, ok ? x : (u32x4)(0u));
        }
        prw = PREFIX ? kc1 - 1 : off + row;
        plw = max(kstart, W > 0 ? max(0, off + row - W + 1) : 0);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) ow[c] = (f32x16)(0.f);
    }

    f32x4 oacc[DB][NBR];
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int nb = 0; nb < NBR; ++nb) oacc[d][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[NBR], l_run[NBR];
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb) {
        m_run[nb] = -INFINITY;
        l_run[nb] = 0.f;
    }

    // ---------------------------------------------------------------- tile copies
    // A plane of a tile is NQ copy instructions of 1 KB: instruction q fills LDS bytes
    // [1024*q, +1024): rows RPI*q + lane / CPR, slot lane % CPR; the IPG instructions of
    // 16-key group ga are q = IPG*ga .. IPG*ga + IPG-1.  Wave w copies only group w % NGA
    // (the first NGA*(nwaves/NGA) waves; the others copy nothing), instructions
    // w / NGA + nsub*j of it, so per tile it looks up one block and forms one base address
    // (kept in scalar registers: the copy address is that base plus a per-lane 32-bit
    // offset fixed for the whole kernel).
    constexpr int IPG = 16 / RPI;          // copy instructions per 16-key group
    const int crow = lane / CPR;           // row within the instruction's rows
    const int cslot = lane % CPR;          // LDS chunk slot within the row
    constexpr int nsub = nwaves / NGA;     // waves per group
    const bool copier = wave < NGA * nsub;
    const int cga = wave % NGA;            // the group this wave copies
    const int csub = wave / NGA;
    // batched: a plane's copies of the group go out under one M0 write (bf16, one wave per
    // group), copy jj at immediate offset 1024*jj; cgk/cgv then hold the lane offsets less that
    // (cg_at adds it back where a copy is issued on its own)
    constexpr bool batched = !FP8 && nsub == 1 && (IPG == 4 || IPG == 2);
    uint32_t cgk[IPG], cgv[IPG];
    int my_copies = 0;                     // copy instructions this wave issues per tile
#pragma unroll
    for (int jj = 0; jj < IPG; ++jj) {
        const int ig = csub + nsub * jj;   // instruction within the group
        const int row = RPI * ig + crow;   // token row within the group (0..15)
        const int ck = cslot ^ (row & KSW);
        const int cv = cslot ^ vswz(row);
        const uint32_t imm = batched ? 1024u * jj : 0u;
        cgk[jj] = (uint32_t)(((row * Hkv + g) * D + ck * 8) * ELT) - imm;
        cgv[jj] = (uint32_t)(((row * Hkv + g) * D + cv * 8) * ELT) - imm;
        my_copies += (copier && ig < IPG) ? 2 : 0;
    }
    auto cg_at = [&](const uint32_t (&cg)[IPG], int jj) -> uint32_t { return cg[jj] + (batched ? 1024u * jj : 0u); };

    // Source of this wave's 16-key group of the tile at k0 (wave-uniform).  A group with no
    // live key takes the rows of the tile's first live group instead, so no block-table entry
    // outside the live range is read.  Keys below `off` come from the cache through the block
    // table; with a fused store, keys from `off` on are the sequence's new tokens and come
    // from the caller's key/value rows (same row layout as a cache plane).  A group that
    // straddles `off` or runs past the last key is copied with per-lane addresses, clamped to
    // the sequence's rows (rows past the last key are zeroed after the copy).
    const char* knew = (const char*)a.knew;
    const char* vnew = (const char*)a.vnew;
    // FUSED: the call stores the new tokens (an FP8 cache is stored by its own kernel first)
    static_assert(!FUSED || (!FP8 && !PREFIX && !CASC), "the fused store is a bf16 prefill of its own");
    constexpr bool fused = FUSED;
    struct GroupSrc {
        const char* k;   // uniform base (non-mixed) of the group's first row, KV head 0
        const char* v;
        int64_t gb;      // cache offset of the group's block rows (mixed groups)
        int j0;          // first key of the group copied
        bool mixed;
    };
    // the group's first key and its block-table entry (looked up apart from forming the
    // addresses, so that the lookup can be issued early)
    struct GroupKey {
        int j0;
        int blk;
        bool mixed;
    };
    auto group_key = [&](int k0) -> GroupKey {
        GroupKey r;
        const int j0 = k0 + 16 * cga;
        const bool live = (j0 <= wg_hi) && (j0 + 15 >= wg_lo);
        r.j0 = live ? j0 : (max(k0, wg_lo) & ~15);
        r.mixed = fused && r.j0 + 15 >= off && (r.j0 < off || r.j0 + 15 > sk - 1);
        r.blk = (!fused || r.j0 < off) ? table[r.j0 >> shift] : 0;
        return r;
    };
    auto group_src_of = [&](const GroupKey& gk) -> GroupSrc {
        GroupSrc r;
        r.j0 = gk.j0;
        r.mixed = gk.mixed;
        r.gb = 0;
        if (!fused || r.j0 < off) {
            // the token's index in the cache fits 32 bits (below num_blocks * block_size)
            r.gb = (int64_t)((uint64_t)(uint32_t)(gk.blk * BS + (r.j0 & (BS - 1))) * (uint32_t)RB);
            r.k = kplane + r.gb;
            r.v = kplane + vdelta + r.gb;
        } else {
            const int64_t row = (int64_t)q0 + r.j0 - off;
            r.k = knew + row * RB;
            r.v = vnew + row * RB;
        }
        return r;
    };
    auto group_src = [&](int k0) -> GroupSrc { return group_src_of(group_key(k0)); };
    // FP8: the codes of the tile in flight, staged until land() widens them into LDS
    u32x2 stg_k[IPG], stg_v[IPG];
    // copy this wave's share of one plane of a tile into LDS buffer dst
    auto issue = [&](const GroupSrc& gs, bool vplane_, const uint32_t (&cg)[IPG], char* dst) {
        if (!copier) return;
        if constexpr (FP8) {
            const char* src = vplane_ ? gs.v : gs.k;
#pragma unroll
            for (int jj = 0; jj < IPG; ++jj) {
                const int ig = csub + nsub * jj;
                if (ig < IPG) (vplane_ ? stg_v : stg_k)[jj] = *(const u32x2*)(src + cg_at(cg, jj));
            }
            return;
        }
        const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst;
        if (!gs.mixed) {
            const char* src = vplane_ ? gs.v : gs.k;
            if constexpr (batched && IPG == 4) {
                copy4_to_lds16<1024>(src, cg, lds + 1024u * (uint32_t)(IPG * cga));
            } else if constexpr (batched && IPG == 2) {
                copy2_to_lds16<1024>(src, cg, lds + 1024u * (uint32_t)(IPG * cga));
            } else {
#pragma unroll
                for (int jj = 0; jj < IPG; ++jj) {
                    const int ig = csub + nsub * jj;
                    if (ig < IPG) copy_to_lds16(src, cg[jj], lds + 1024u * (uint32_t)(IPG * cga + ig));
                }
            }
        } else {
#pragma unroll
            for (int jj = 0; jj < IPG; ++jj) {
                const int ig = csub + nsub * jj;
                if (ig < IPG) {
                    const int row = RPI * ig + crow;
                    const int key = gs.j0 + row;
                    const char* p;
                    if (key < off) {
                        p = kplane + (vplane_ ? vdelta : 0) + gs.gb + cg_at(cg, jj);
                    } else {
                        const int64_t rn = (int64_t)q0 + min(key, sk - 1) - off;
                        p = (vplane_ ? vnew : knew) + rn * RB + (cg_at(cg, jj) - (uint32_t)row * (uint32_t)RB);
                    }
                    copy_to_lds16_lane(p, lds + 1024u * (uint32_t)(IPG * cga + ig));
                }
            }
        }
    };
    // FP8: widen the staged codes of this wave's share of a tile into its LDS buffers
    auto land = [&](char* dk, char* dv) {
        if (!copier) return;
        auto widen = [](u32x2 w) {
            return u32x4{e4m3x2_to_bf16(w[0], false), e4m3x2_to_bf16(w[0], true), e4m3x2_to_bf16(w[1], false),
                         e4m3x2_to_bf16(w[1], true)};
        };
#pragma unroll
        for (int jj = 0; jj < IPG; ++jj) {
            const int ig = csub + nsub * jj;
            if (ig < IPG) {
                const uint32_t o = 1024u * (uint32_t)(IPG * cga + ig) + 16u * lane;
                *(u32x4*)(dk + o) = widen(stg_k[jj]);
                *(u32x4*)(dv + o) = widen(stg_v[jj]);
            }
        }
    };
    // after this wave's copies of a plane of the tile at k0 landed: zero the rows it copied
    // whose key lies outside [wg_lo, wg_hi]
    auto zero_dead = [&](int k0, char* dst) {
        if (!copier || (k0 >= wg_lo && k0 + BN - 1 <= wg_hi)) return;
#pragma unroll
        for (int jj = 0; jj < IPG; ++jj) {
            const int ig = csub + nsub * jj;
            if (ig < IPG) {
                const int key = k0 + 16 * cga + RPI * ig + crow;
                if (key < wg_lo || key > wg_hi)
                    *(u32x4*)(dst + 1024 * (IPG * cga + ig) + 16 * lane) = (u32x4)(0u);
            }
        }
    };

    // LDS operand addresses of this lane: K row 16*ga + col, chunk (4t + grp) swizzled by
    // the row, and (16*ga + col) & KSW == col & KSW, so only the 16*ga row offset depends on ga
    uint32_t koff[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) koff[t] = (uint32_t)(col * D * 2 + (((4 * t + grp) ^ (col & KSW)) * 16));
    // V^T: source lane col of group grp addresses row 32cc + 16hh + 4*grp + col/4, dims
    // 16*db + 4*(col%4) .. +4; the row's swizzle depends on (row & 7) = (4*grp + col/4) & 7
    const int vrow0 = 4 * grp + (col >> 2);
    const int vsw = vswz(vrow0);
    const uint32_t voff_base = (uint32_t)(vrow0 * D * 2 + 8 * (col & 1));
    const int vch = (col & 3) >> 1;  // chunk within the 16-dim block

    // S^T of the tile whose K sits at kbuf
    auto qk = [&](const char* kt, f32x4 (&sacc)[NGA][NBR]) {
#pragma unroll
        for (int ga = 0; ga < NGA; ++ga)
#pragma unroll
            for (int nb = 0; nb < NBR; ++nb) sacc[ga][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KS; ++t) {
#pragma unroll
            for (int ga = 0; ga < NGA; ++ga) {
                const bf16x8 kf = *(const bf16x8*)(kt + koff[t] + 16 * ga * D * 2);
#pragma unroll
                for (int nb = 0; nb < NBR; ++nb)
                    sacc[ga][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nb][t], sacc[ga][nb], 0, 0, 0);
            }
        }
    };

    // mask, online softmax, P^T pack; returns whether O needs rescaling
    auto softmax = [&](int k0, f32x4 (&sacc)[NGA][NBR], u32x4 (&pk)[NCC][NBR], float (&alpha)[NBR]) {
        const bool edge = (k0 + BN - 1 > wv_p_min) || (has_lo && k0 < wv_lo_max);
        if (edge) {
#pragma unroll
            for (int ga = 0; ga < NGA; ++ga)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + 16 * ga + 4 * grp + r;
#pragma unroll
                    for (int nb = 0; nb < NBR; ++nb)
                        sacc[ga][nb][r] = (key > prow[nb] || key < plo[nb]) ? -INFINITY : sacc[ga][nb][r];
                }
        }
        // cs: factor from the accumulator to log2 units (1 once ALiBi has folded it in)
        float cs = c_log2;
        if constexpr (ALIBI) {
#pragma unroll
            for (int nb = 0; nb < NBR; ++nb) {
                const float base = sl2 * (float)(k0 + 4 * grp - prow[nb]);
#pragma unroll
                for (int ga = 0; ga < NGA; ++ga)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sacc[ga][nb][r] = fmaf(sacc[ga][nb][r], c_log2, fmaf(sl2, (float)(16 * ga + r), base));
            }
            cs = 1.f;
        }
#pragma unroll
        for (int nb = 0; nb < NBR; ++nb) {
            // three-operand chain: one v_max3 per two scores
            float mx = fmaxf(sacc[0][nb][0], sacc[0][nb][1]);
#pragma unroll
            for (int x = 2; x < 4 * NGA; x += 2)
                mx = fmaxf(fmaxf(mx, sacc[x >> 2][nb][x & 3]), sacc[x >> 2][nb][(x & 3) + 1]);
            mx = group4_max(mx);
            // The reference maximum moves only when the tile's maximum exceeds it by more
            // than 8 (log2 units): P = exp2(s - m) then stays below 2^8, and O and l are
            // rescaled only on those rare moves instead of on every increase.
            const float mt = mx * cs;
            const bool move = mt > m_run[nb] + 8.f;
            const float m_new = move ? mt : m_run[nb];
            alpha[nb] = (move && m_run[nb] != -INFINITY) ? __builtin_amdgcn_exp2f(m_run[nb] - m_new) : 1.f;
            m_run[nb] = m_new;
            const float msub = m_new == -INFINITY ? 0.f : m_new;
            float pv[NGA][4];
#pragma unroll
            for (int ga = 0; ga < NGA; ++ga)
#pragma unroll
                for (int r = 0; r < 4; ++r) pv[ga][r] = __builtin_amdgcn_exp2f(fmaf(sacc[ga][nb][r], cs, -msub));
            float ps = 0.f;
#pragma unroll
            for (int ga = 0; ga < NGA; ++ga) ps += (pv[ga][0] + pv[ga][1]) + (pv[ga][2] + pv[ga][3]);
            l_run[nb] = l_run[nb] * alpha[nb] + ps;
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) {
                pk[cc][nb][0] = pack_bf16x2(pv[2 * cc][0], pv[2 * cc][1]);
                pk[cc][nb][1] = pack_bf16x2(pv[2 * cc][2], pv[2 * cc][3]);
                pk[cc][nb][2] = pack_bf16x2(pv[2 * cc + 1][0], pv[2 * cc + 1][1]);
                pk[cc][nb][3] = pack_bf16x2(pv[2 * cc + 1][2], pv[2 * cc + 1][3]);
            }
        }
    };

    auto pv_mfma = [&](const char* vt, const u32x4 (&pk)[NCC][NBR], const float (&alpha)[NBR]) {
        bool rescale = false;
#pragma unroll
        for (int nb = 0; nb < NBR; ++nb) rescale = rescale || alpha[nb] != 1.f;
        if (__any(rescale)) {
#pragma unroll
            for (int d = 0; d < DB; ++d)
#pragma unroll
                for (int nb = 0; nb < NBR; ++nb) oacc[d][nb] *= alpha[nb];
        }
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            bf16x8 vf[DB];
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                s16x4 vh[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int rowoff = (32 * cc + 16 * hh) * D * 2;  // rows shift by 16: same swizzle
                    const uint32_t o = voff_base + rowoff + (((2 * d + vch) ^ vsw) * 16);
                    vh[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) char*)vt + o));
                }
                vf[d] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int d = 0; d < DB; ++d)
#pragma unroll
                for (int nb = 0; nb < NBR; ++nb)
                    oacc[d][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        vf[d], __builtin_bit_cast(bf16x8, pk[cc][nb]), oacc[d][nb], 0, 0, 0);
        }
    };

    // ---------------------------------------------------------------- 32x32x16 form
    // K operand of lane l: tile row 32b + l % 32, 16-byte chunk 2t + l / 32 (swizzled by the
    // row; (32b + l % 32) & KSW == l & KSW)
    uint32_t kw[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) kw[t] = (uint32_t)(lrow * D * 2 + (((2 * t + lh) ^ (lrow & KSW)) * 16));
    auto qk_w = [&](const char* kt, f32x16 (&sw)[NB32], int k0) {
        if constexpr (ALIBI) {
            // bias of key k0 + 32b + 8(i/4) + 4(l/32) + i%4 for this lane's row, over the scale
            const float base = sl2r * (float)(k0 + 4 * lh - prw);
#pragma unroll
            for (int b = 0; b < NB32; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) sw[b][i] = fmaf(sl2r, (float)(32 * b + 8 * (i >> 2) + (i & 3)), base);
        } else {
#pragma unroll
            for (int b = 0; b < NB32; ++b) sw[b] = (f32x16)(0.f);
        }
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
#pragma unroll
            for (int b = 0; b < NB32; ++b) {
                const bf16x8 kf = *(const bf16x8*)(kt + kw[t] + 32 * b * D * 2);
                sw[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qw[t], sw[b], 0, 0, 0);
            }
        // operand reads well ahead of their MFMAs (the default order issued them one or two
        // MFMAs ahead, less than the LDS latency): eight first, then one per MFMA
        constexpr int NR = NB32 * (D / 16);
#pragma unroll
        for (int r = 0; r < 8; ++r) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int m = 0; m < NR; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (m + 8 < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    // mask, online softmax of the lane's row, P^T packed straight from the accumulators: the
    // B operand of 16-key step (b, sg) is accumulator values 8 sg .. 8 sg + 7 of block b
    auto softmax_w = [&](int k0, f32x16 (&sw)[NB32], u32x4 (&pw)[NB32][2], float& alpha, bool inner) {
        const bool edge = !inner && ((k0 + CB - 1 > wv_p_min) || (has_lo && k0 < wv_lo_max));
        if (edge) {
#pragma unroll
            for (int b = 0; b < NB32; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 32 * b + 8 * (i >> 2) + 4 * lh + (i & 3);
                    sw[b][i] = (key > prw || key < plw) ? -INFINITY : sw[b][i];
                }
        }
        const float cs = c_log2;  // (ALiBi: the bias is already in the accumulators)
        float mx = fmaxf(sw[0][0], sw[0][1]);
#pragma unroll
        for (int x = 2; x < 16 * NB32; x += 2) mx = fmaxf(fmaxf(mx, sw[x >> 4][x & 15]), sw[x >> 4][(x & 15) + 1]);
        mx = half_max(mx);
        // the reference maximum moves only when the tile's maximum exceeds it by more than 8
        // (log2 units), as in the 16x16 form
        const float mt = mx * cs;
        const bool move = mt > mw + 8.f;
        const float m_new = move ? mt : mw;
        alpha = (move && mw != -INFINITY) ? __builtin_amdgcn_exp2f(mw - m_new) : 1.f;
        mw = m_new;
        const float msub = m_new == -INFINITY ? 0.f : m_new;
        float ps = 0.f;
#pragma unroll
        for (int b = 0; b < NB32; ++b)
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                float pv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) pv[j] = __builtin_amdgcn_exp2f(fmaf(sw[b][8 * sg + j], cs, -msub));
                ps += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
                pw[b][sg] = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                                  pack_bf16x2(pv[6], pv[7])};
            }
        lw = lw * alpha + ps;
    };
    // V^T operand of lane l for dims 32c + l % 32 and 16-key step rb: two transposing LDS reads
    // per 16-lane group g: source lane s addresses row rb + 4 * (g / 2) + s / 4 (+ 8 for the
    // second), dims 32c + 16 * (g % 2) + 4 * (s % 4); lane i of the group receives the four
    // consecutive keys at dim 32c + 16 * (g % 2) + i, i.e. keys rb + 4 * (l / 32) + 0..3 (and
    // + 8) at dim 32c + l % 32 -- the key order of the P^T operand
    const int vgw = lane >> 4;
    const int vsl = lane & 15;
    const int vroww = 4 * (vgw >> 1) + (vsl >> 2);
    const uint32_t vbasew = (uint32_t)(vroww * D * 2 + 8 * (vsl & 1));
    const int vsww = vswz(vroww);  // rows shifted by multiples of 4: same swizzle
    auto pv_w = [&](const char* vt, const u32x4 (&pw)[NB32][2], float alpha) {
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int c = 0; c < D / 32; ++c) ow[c] *= alpha;
        }
#pragma unroll
        for (int b = 0; b < NB32; ++b)
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                const uint32_t rowoff = (uint32_t)((32 * b + 16 * sg) * D * 2);
#pragma unroll
                for (int c = 0; c < D / 32; ++c) {
                    const uint32_t chunk = (uint32_t)(4 * c + 2 * (vgw & 1) + ((vsl >> 1) & 1));
                    const uint32_t o = vbasew + rowoff + ((chunk ^ (uint32_t)vsww) * 16);
                    typedef __attribute__((address_space(3))) char lchar;
                    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lchar*)vt + o));
                    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lchar*)vt + o + 8 * D * 2));
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                    ow[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, pw[b][sg]), ow[c], 0, 0, 0);
                }
            }
        // V operand reads ahead of their MFMAs as for K: eight first (four MFMAs' worth), then two
        // per MFMA
        constexpr int NM = 2 * NB32 * (D / 32);
#pragma unroll
        for (int r = 0; r < 8; ++r) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (m + 4 < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
    };

    // ---------------------------------------------------------------- fused store
    // A new token's K/V rows reach LDS in the tiles around the diagonal of the q-tile that
    // holds its query row.  In those steps the workgroup that holds the pair (row block, head
    // 0) of the row writes the row (KV head g's part, both planes) from LDS to its cache slot
    // (negative slots skipped): no extra global read, and the stores overlap the math.  The
    // attention never reads these cache rows (it takes new keys from the caller's rows).
    // the q-tile's slots, staged in LDS once (a global load inside the loop would make the
    // compiler wait for every copy in flight); filled right after the first tile's copies are
    // issued, so its wait overlaps theirs
    __shared__ int lds_slots[32 * kPrefillWaves];  // 32 rows per row block, rb <= waves
    auto stage_slots = [&]() {
        for (int i = tid; i < 32 * pg.rb; i += blockDim.x)
            lds_slots[i] = i0 + i < sq ? a.slots[q0 + i0 + i] : -1;
    };
    auto store_new_rows = [&](int k0, const char* kc, const char* vc) {
        const int ks = max(k0, off + wg_row0);
        const int ke = min(k0 + BN, off + wg_row_end);
        if (ks >= ke) return;
        constexpr int CH = D * 2 / 16;  // 16-byte chunks per row and plane
        for (int idx = tid; idx < (ke - ks) * CH; idx += blockDim.x) {
            const int key = ks + idx / CH;
            const int c = idx % CH;
            const int i = key - off;                           // query row of the token
            if (((i - i0) / 32 * G) / kPrefillWaves != jw) continue;  // another workgroup's row block
            const int slot = lds_slots[i - i0];
            if (slot < 0) continue;
            const int r = key - k0;                            // row in the tile
            const u32x4 kx = *(const u32x4*)(kc + r * D * 2 + ((c ^ (r & KSW)) * 16));
            const u32x4 vx = *(const u32x4*)(vc + r * D * 2 + ((c ^ vswz(r)) * 16));
            const int64_t dst = ((int64_t)slot * Hkv + g) * D * 2 + c * 16;
            *(u32x4*)((char*)a.c.kv + dst) = kx;
            *(u32x4*)((char*)a.c.kv + vdelta + dst) = vx;
        }
    };

    // ---------------------------------------------------------------- main loop
    // A ring of NBUF buffer pairs: while tile kt computes, the copies of tiles kt+1 ..
    // kt+NBUF-1 are in flight.  Tile kt sits in buffer (kt - kt_begin) % NBUF; the loop body
    // is written out NBUF times so each step names fixed buffers.
    auto kbuf = [&](auto J) -> char* {
        constexpr int j = decltype(J)::value;
        return j == 0 ? lds_k0 : j == 1 ? lds_k1 : j == 2 ? lds_k2 : lds_k3;
    };
    auto vbuf = [&](auto J) -> char* {
        constexpr int j = decltype(J)::value;
        return j == 0 ? lds_v0 : j == 1 ? lds_v1 : j == 2 ? lds_v2 : lds_v3;
    };
    // Inner tiles [ia, ib): tiles every row of the workgroup sees in full, from the last
    // first-key of its rows up to below its first row's own position (PREFIX: the chunk's
    // whole tiles).  They need no mask and hold no dead rows, every active wave computes them,
    // and they hold none of the workgroup's own new tokens: one test per tile skips those checks.
    const int lo_all = PREFIX ? kc0 : max(kstart, W > 0 ? max(0, off + wg_row_end - W) : 0);
    const int hi_all = PREFIX ? kc1 - 1 : off + wg_row0 - 1;
    const int ia = (lo_all + BN - 1) / BN;
    const int ib = (hi_all + 1) / BN;
    auto step = [&](int kt, int kt_end, auto J) {
        constexpr int j = decltype(J)::value;
        const bool inner = kt >= ia && kt < ib;
        constexpr int jn = (j + NBUF - 1) % NBUF;  // buffer of tile kt + NBUF - 1
        char* kc = kbuf(J);
        char* vc = vbuf(J);
        const int k0 = kt * BN;
        // the group this step copies (tile kt + NBUF - 1; tile kt's own when there is none, a
        // lookup already made), its block-table entry loaded before the waits below
        const bool has_next = kt + NBUF - 1 < kt_end;
        const GroupKey gk = group_key((has_next ? kt + NBUF - 1 : kt) * BN);
        // this wave's copies of tile kt have landed once at most those of the tiles after
        // it (up to NBUF - 2 of them) are still in flight
        if constexpr (FP8) {
            land(kc, vc);  // the compiler waits for the staged loads it issued
        } else {
            const int later = min(NBUF - 2, kt_end - 1 - kt);
            wait_vmcnt(my_copies * later);
        }
        if (!inner) {
            zero_dead(k0, kc);
            zero_dead(k0, vc);
        }
        // all copies of tile kt visible; buffer jn (tile kt - 1) is free.  Not a fenced
        // barrier: that would also wait for the copies of the later tiles
        lds_barrier_after(gk.blk);
        if (has_next) {
            const GroupSrc gs = group_src_of(gk);
            issue(gs, false, cgk, kbuf(std::integral_constant<int, jn>{}));
            issue(gs, true, cgv, vbuf(std::integral_constant<int, jn>{}));
        }
        if (!inner && fused) store_new_rows(k0, kc, vc);
        if (inner ? wave_active : (wave_active && k0 <= wv_hi && k0 + BN - 1 >= wv_lo)) {
            if constexpr (W32) {
#pragma unroll
                for (int hb = 0; hb < BN / CB; ++hb) {
                    f32x16 sw[NB32];
                    u32x4 pw[NB32][2];
                    float alpha;
                    qk_w(kc + hb * CB * D * 2, sw, k0 + hb * CB);
                    softmax_w(k0 + hb * CB, sw, pw, alpha, inner);
                    pv_w(vc + hb * CB * D * 2, pw, alpha);
                }
            } else {
                f32x4 sacc[NGA][NBR];
                u32x4 pk[NCC][NBR];
                float alpha[NBR];
                qk(kc, sacc);
                softmax(k0, sacc, pk, alpha);
                pv_mfma(vc, pk, alpha);
            }
        }
    };
    // a buffer pair no wave reads after the loop (the one before the last tile's; any when
    // there is a single tile or none): the epilogue stages the output tiles there
    int free_buf = 1;
    if (wg_hi >= wg_lo) {
        const int kt_begin = wg_lo / BN;
        const int kt_end = wg_hi / BN + 1;
        free_buf = (kt_end - 1 - kt_begin + NBUF - 1) % NBUF;
        {
            GroupSrc gs = group_src(kt_begin * BN);
            issue(gs, false, cgk, lds_k0);
            issue(gs, true, cgv, lds_v0);
            if (NBUF > 2 && kt_begin + 1 < kt_end) {
                gs = group_src((kt_begin + 1) * BN);
                issue(gs, false, cgk, lds_k1);
                issue(gs, true, cgv, lds_v1);
            }
            if (NBUF > 3 && kt_begin + 2 < kt_end) {
                gs = group_src((kt_begin + 2) * BN);
                issue(gs, false, cgk, lds_k2);
                issue(gs, true, cgv, lds_v2);
            }
        }
        if (fused) stage_slots();
        for (int kt = kt_begin; kt < kt_end; kt += NBUF) {
            step(kt, kt_end, std::integral_constant<int, 0>{});
            if (kt + 1 < kt_end) step(kt + 1, kt_end, std::integral_constant<int, 1>{});
            if constexpr (NBUF > 2)
                if (kt + 2 < kt_end) step(kt + 2, kt_end, std::integral_constant<int, 2>{});
            if constexpr (NBUF > 3)
                if (kt + 3 < kt_end) step(kt + 3, kt_end, std::integral_constant<int, 3>{});
        }
    }

    // ---------------------------------------------------------------- epilogue
    if (!wave_active) return;
    if constexpr (W32) {
        const float lt = half_sum(lw);  // before any lane leaves: both halves of the row
        const int row = r0 + lrow;
        if constexpr (!PREFIX) {
            // bf16 output: the wave's 32 x D tile goes through its 32 rows x 2D bytes of the free
            // buffer (row-major, 16-byte chunk c of row r at slot c ^ (r & KSW)), so that each
            // global store writes whole rows (the accumulator layout would store 8-byte pieces
            // of 32 rows per instruction)
            float lsum = lt;
            if constexpr (CASC) {
                // the prefix pass's states of this packed row and head (one per prefix chunk),
                // folded in by log-sum-exp: both parts are in the same log2 units
                if (row < rows_end) {
                    const int64_t per_chunk = (int64_t)a.prefix_rows * H;
                    const int64_t st = (int64_t)(q0 + row) * H + h;
                    float M = mw;
                    for (int c = 0; c < a.prefix_chunks; ++c) M = fmaxf(M, a.pre_ml[(c * per_chunk + st) * 2]);
                    const float msub = M == -INFINITY ? 0.f : M;
                    const float al = __builtin_amdgcn_exp2f(mw - msub);
                    lsum *= al;
#pragma unroll
                    for (int c = 0; c < D / 32; ++c) ow[c] *= al;
                    for (int c = 0; c < a.prefix_chunks; ++c) {
                        const f32x2 ml = *(const f32x2*)(a.pre_ml + (c * per_chunk + st) * 2);
                        const float w = __builtin_amdgcn_exp2f(ml[0] - msub);
                        lsum = fmaf(w, ml[1], lsum);
                        const float* po = a.pre_o + (c * per_chunk + st) * D + 4 * lh;
#pragma unroll
                        for (int cc = 0; cc < D / 32; ++cc)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const f32x4 x = *(const f32x4*)(po + 32 * cc + 8 * q);
#pragma unroll
                                for (int e = 0; e < 4; ++e) ow[cc][4 * q + e] = fmaf(w, x[e], ow[cc][4 * q + e]);
                            }
                    }
                }
            }
            const float inv = lsum > 0.f ? (FP8 ? a.c.kv_scale : 1.f) / lsum : 0.f;  // FP8: V / kv_scale in the cache
            constexpr int TW = 32 * D * 2;  // bytes of one wave's output tile
            static_assert(kPrefillWaves * TW <= 2 * TILE, "the free buffer pair holds every wave's output tile");
            char* stg = (free_buf == 0 ? lds_k0 : free_buf == 1 ? lds_k1 : free_buf == 2 ? lds_k2 : lds_k3);
            if (wave >= TILE / TW) stg = (free_buf == 0 ? lds_v0 : free_buf == 1 ? lds_v1 : free_buf == 2 ? lds_v2 : lds_v3);
            stg += (wave % (TILE / TW)) * TW;
            // lane (row lrow, half lh) holds dims 32c + 8q + 4lh .. +3: 16-byte chunk 4c + q, half lh
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(u32x2*)(stg + lrow * D * 2 + (((4 * c + q) ^ (lrow & KSW)) * 16) + 8 * lh) =
                        u32x2{pack_bf16x2(ow[c][4 * q] * inv, ow[c][4 * q + 1] * inv),
                              pack_bf16x2(ow[c][4 * q + 2] * inv, ow[c][4 * q + 3] * inv)};
            // read back whole rows: lane l takes chunk l % CPR of row RPI * k + l / CPR
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const int rr = RPI * k + lane / CPR;
                const int ch = lane % CPR;
                const u32x4 x = *(const u32x4*)(stg + rr * D * 2 + ((ch ^ (rr & KSW)) * 16));
                if (r0 + rr < rows_end)
                    *(u32x4*)((__bf16*)a.out + ((int64_t)(q0 + r0 + rr) * H + h) * D + 8 * ch) = x;
            }
            return;
        }
        if (row >= rows_end) return;
        if constexpr (PREFIX) {
            const int64_t st = ((int64_t)pc * a.num_seqs + row) * H + h;
            float* po = a.pre_o + st * D + 4 * lh;
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(f32x4*)(po + 32 * c + 8 * q) = f32x4{ow[c][4 * q], ow[c][4 * q + 1], ow[c][4 * q + 2], ow[c][4 * q + 3]};
            if (lh == 0) *(f32x2*)(a.pre_ml + st * 2) = f32x2{mw, lt};
            return;
        }
    }
    if constexpr (PREFIX) {  // the chunk's state of each (row, head): O, running max, sum
#pragma unroll
        for (int nb = 0; nb < NBR; ++nb) {
            const float lt = group4_sum(l_run[nb]);
            const int row = r0 + 16 * nb + col;
            if (row >= rows_end) continue;
            const int64_t st = ((int64_t)pc * a.num_seqs + row) * H + h;
            float* po = a.pre_o + st * D + 4 * grp;
#pragma unroll
            for (int d = 0; d < DB; ++d) *(f32x4*)(po + 16 * d) = oacc[d][nb];
            if (grp == 0) *(f32x2*)(a.pre_ml + st * 2) = f32x2{m_run[nb], lt};
        }
        return;
    }
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb) {
        const float lt = group4_sum(l_run[nb]);
        const int row = r0 + 16 * nb + col;
        if (row >= rows_end) continue;
        const float inv = lt > 0.f ? (FP8 ? a.c.kv_scale : 1.f) / lt : 0.f;  // FP8: V / kv_scale in the cache
        __bf16* dst = (__bf16*)a.out + ((int64_t)(q0 + row) * H + h) * D + 4 * grp;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
            const f32x4 o = oacc[d][nb];
            *(u32x2*)(dst + 16 * d) = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
        }
    }
}

// Launch shape: keys per K/V tile and K/V buffers in the copy ring.
constexpr int kPrefillBN = 64;
constexpr int kPrefillNBUF = 2;
// MFMA form of the attention contraction: 32x32x16 (true) or 16x16x32 (false).  Measured on
// the 16-prompt causal batch, the chunked-window and the mixed prefills: 32x32x16 1-3% faster
// with 18 fewer VGPRs.
constexpr bool kPrefillW32 = true;
// every 16-key group of a tile needs a wave of its own to copy it
static_assert(kPrefillBN / 16 <= kPrefillWaves, "fewer waves than key groups per tile");

static int gcd_int(int x, int y) {
    while (y) {
        const int t = x % y;
        x = y;
        y = t;
    }
    return x;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t st) {
    const int G = a.group;
    // 32 query rows per wave, kPrefillWaves waves per workgroup, 8 waves per CU (measured: two
    // independent 4-wave workgroups per CU beat one workgroup of 5..8 waves)
    PrefillGrid pg;
    pg.rb = kPrefillWaves / gcd_int(G, kPrefillWaves);
    pg.wgs_per_tile = G * pg.rb / kPrefillWaves;
    pg.n_sg = a.num_seqs * a.c.num_kv_heads;
    pg.n_tiles = (a.max_seqlen_q + 32 * pg.rb - 1) / (32 * pg.rb) * pg.wgs_per_tile;
    const int64_t nsg_pad = ((int64_t)pg.n_sg + 7) / 8 * 8;
    const dim3 grid((unsigned)(nsg_pad * pg.n_tiles));
    const bool alibi = a.alibi != nullptr;
    const bool fp8 = a.c.dtype == 2;
    const bool fused = a.knew != nullptr;  // bf16 only: the FP8 path stores first
#define PA_PREFILL(DD, AL, F8, FU) hipLaunchKernelGGL((prefill_bf16_kernel<DD, 2, kPrefillBN, (F8 ? 2 : kPrefillNBUF), AL, F8, false, kPrefillW32, false, FU>), grid, dim3(64 * kPrefillWaves), 0, st, a, pg)
#define PA_PREFILL_BF16(DD, AL) do { if (fused) PA_PREFILL(DD, AL, false, true); else PA_PREFILL(DD, AL, false, false); } while (0)
#define PA_CASC(DD, F8) hipLaunchKernelGGL((prefill_bf16_kernel<DD, 2, kPrefillBN, (F8 ? 2 : kPrefillNBUF), false, F8, false, true, true, false>), grid, dim3(64 * kPrefillWaves), 0, st, a, pg)
    if (fused && (fp8 || a.cascade)) return hipErrorInvalidValue;
    if (a.cascade) {  // shared-prefix own-keys pass (no ALiBi, no fused store)
        if (a.c.head_size == 128) { if (fp8) PA_CASC(128, true); else PA_CASC(128, false); }
        else { if (fp8) PA_CASC(64, true); else PA_CASC(64, false); }
    } else if (a.c.head_size == 128) {
        if (fp8) { if (alibi) PA_PREFILL(128, true, true, false); else PA_PREFILL(128, false, true, false); }
        else { if (alibi) PA_PREFILL_BF16(128, true); else PA_PREFILL_BF16(128, false); }
    } else {
        if (fp8) { if (alibi) PA_PREFILL(64, true, true, false); else PA_PREFILL(64, false, true, false); }
        else { if (alibi) PA_PREFILL_BF16(64, true); else PA_PREFILL_BF16(64, false); }
    }
#undef PA_PREFILL_BF16
#undef PA_PREFILL
#undef PA_CASC
    return hipGetLastError();
}

// q-tile pairs of the prefill grid for group size G (rb row blocks of 32 per q-tile)
static PrefillGrid prefix_grid(int num_seqs, int group, int num_kv_heads, int chunks) {
    PrefillGrid pg;
    pg.rb = kPrefillWaves / gcd_int(group, kPrefillWaves);
    pg.wgs_per_tile = group * pg.rb / kPrefillWaves;
    pg.n_sg = chunks * num_kv_heads;
    pg.n_tiles = (num_seqs + 32 * pg.rb - 1) / (32 * pg.rb) * pg.wgs_per_tile;
    return pg;
}

int prefix_tiles(int prefix_len) { return (prefix_len + kPrefillBN - 1) / kPrefillBN; }

int prefix_workgroups_per_chunk(int num_seqs, int group, int num_kv_heads) {
    return prefix_grid(num_seqs, group, num_kv_heads, 1).n_tiles * num_kv_heads;
}

hipError_t launch_prefix_states(const DecodeArgs& d, hipStream_t st) {
    PrefillArgs a;
    a.c = d.c;
    a.out = nullptr;
    a.q = d.q;
    a.table = d.table;  // row 0: the prefix blocks every row shares
    a.max_blocks = d.max_blocks;
    a.cu_q = nullptr;
    a.cu_k = nullptr;
    a.num_seqs = d.num_seqs;
    a.max_seqlen_q = d.num_seqs;
    a.num_heads = d.num_heads;
    a.group = d.group;
    a.scale = d.scale;
    a.window = 0;
    a.knew = nullptr;
    a.vnew = nullptr;
    a.slots = nullptr;
    a.alibi = nullptr;
    a.prefix_len = d.key_start;
    a.prefix_chunks = d.prefix_chunks;
    a.pre_o = d.pre_o;
    a.pre_ml = d.pre_ml;
    a.cascade = 0;
    a.prefix_rows = d.num_seqs;
    const PrefillGrid pg = prefix_grid(d.num_seqs, d.group, d.c.num_kv_heads, d.prefix_chunks);
    const int64_t nsg_pad = ((int64_t)pg.n_sg + 7) / 8 * 8;
    const dim3 grid((unsigned)(nsg_pad * pg.n_tiles));
    const bool fp8 = a.c.dtype == 2;
#define PA_PREFIX(DD, F8) hipLaunchKernelGGL((prefill_bf16_kernel<DD, 2, kPrefillBN, (F8 ? 2 : kPrefillNBUF), false, F8, true, kPrefillW32, false, false>), grid, dim3(64 * kPrefillWaves), 0, st, a, pg)
    if (a.c.head_size == 128) {
        if (fp8) PA_PREFIX(128, true); else PA_PREFIX(128, false);
    } else {
        if (fp8) PA_PREFIX(64, true); else PA_PREFIX(64, false);
    }
#undef PA_PREFIX
    return hipGetLastError();
}

}  // namespace pa
