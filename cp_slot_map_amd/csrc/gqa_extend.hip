// bf16 GQA attention of many query rows per kv head (head_dim = head_dim_v = 128), built for gfx950 MFMA: the
// per-stripe partial of rows that bring several tokens in a step (context part), and the causal attention of a row's
// in-step tokens over one another (own-token part).
//
// What it computes. Context part: each query token of a row attends the stripe's prior context positions and the
// partial is returned with its natural-log lse (mstar PR #1124, "Context / Sequence Parallel 1/5", PR description;
// every in-step query sees the whole prior context). Own-token part: query i of a row attends the row's in-step keys
// 0..i, taken from the K/V the layer hands over (same PR; the own-token call in the vLLM compare view
// "[Core] Add explicit layer parallel plans" passes the query offsets as the key offsets).
//
// Work decomposition. A unit is (row b, stripe s, kv head g, block of 128 query rows); query rows of a kv head are
// (token, head-in-group) pairs, so a block holds 128 / G tokens. One workgroup of four waves (one per SIMD) runs a
// unit and two workgroups share a CU, so that one workgroup's softmax overlaps the other's matrix products; wave w
// owns rows [32w, 32w + 32) as two MFMA row blocks and keeps their query operand (32 VGPRs) and output accumulators
// (64 VGPRs) in registers. K and V stream through LDS in tiles of 32 tokens (16 KB; four buffers, three tiles in
// flight), loaded straight from global memory into LDS: each wave issues two K and two V instructions per tile, 64
// lanes covering four tokens' 256-byte rows. Every K read and every V read from LDS serves both row blocks of the
// wave, so the LDS traffic per MFMA is a quarter of what a 16-row wave would need.
//
// Per tile and wave (32 rows x 32 tokens):
//   * scores S^T[token][row] = K . Q^T with v_mfma_f32_16x16x32_bf16 (16 MFMAs): A = K rows from LDS, B = query rows.
//   * softmax against a fixed per-row reference (the maximum of the unit's first tile; the scale enters each exponent
//     through one fused multiply-add; row maxima and sums over the four lane groups use the gfx950 lane swaps); keys
//     past the end and, in the own-token part, keys after the query's own token are masked (only on the tiles that
//     reach them).
//   * out += P . V with v_mfma_f32_16x16x32_f16: the score layout is the A-operand layout (k index 8c + e of lane
//     group c is tile token 16 (e / 4) + 4c + e % 4), the B operand of a 16-dim output tile comes from two transposed
//     LDS reads (ds_read_b64_tr_b16) widened from bf16 to fp16 in registers (exact: value magnitudes must stay below
//     65504). P enters rounded to fp16 (11 significant bits) and each row is normalised by the sum of exactly those
//     rounded weights, so they sum to one; one bf16 rounding of P (8 bits) put a softmax peaked on a few keys past
//     2e-3 of the float64 result, and the earlier bf16 pair (hi + residual, 16 bits) took twice the MFMAs (16 MFMAs).
//
// LDS layout of a tile: K rows of 256 bytes at 256 t, V rows at 8192 + 256 t; the sixteen 16-byte pieces of token t
// are stored XOR f(t) = 2t mod 16. Measured on gfx950, the score reads (sixteen tokens at one piece) and the transposed
// value reads then run at the full rate of their instruction; without the swizzle they run at an eighth of it.
//
// fp8 pools (context part): a wave's 8 tokens of K codes (128 bytes a token) arrive with one direct-to-LDS instruction
// in the upper half of the wave's K rows, and likewise for V; once they have landed the loading wave widens them in
// place, K to bf16 and V to fp16 (both exact for every E4M3 code), into the same swizzled rows, so the products read
// the same operands as over bf16 pools. The key descale is folded into the score scale and the value descale into the
// output normalisation, both in fp32.
#include "launch.h"

#include <type_traits>

namespace cpattn {

namespace {

constexpr int kD = 128;
constexpr int kTile = 32;                       // keys per LDS tile
constexpr int kRowBytes = kD * 2;               // one token's K (or V) row
constexpr int kVOff = kTile * kRowBytes;        // V region of a tile
constexpr int kTileBytes = 2 * kTile * kRowBytes;
constexpr int kBufs = 4;
constexpr int kAhead = kBufs - 1;
constexpr int kNW = 4;                          // waves per workgroup (two workgroups per CU)
constexpr int kRowsPerWave = 32;
constexpr int kBlockRows = kNW * kRowsPerWave;  // query rows per unit
constexpr int kMaxPages = 2048;                 // page ids of a stripe staged in LDS
constexpr int kMaxPlanTriples = 8192;           // (row, stripe, query block) triples the plan kernel ranks
constexpr int kTokPerWave = kTile / kNW;        // tokens of a tile each wave loads
// Direct-to-LDS instructions per wave and tile (K and V): 1 KB each, so four tokens of bf16 rows or eight of fp8 rows.
template <bool KV8>
constexpr int loads_per_tile() { return KV8 ? 2 : 2 * (kTokPerWave / 4); }
constexpr int kStage8 = kTokPerWave * kRowBytes / 2;   // fp8 codes of a wave's tokens: upper half of its rows

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) char* lds_char_ptr;
typedef const __attribute__((address_space(3))) int32_t* lds_i32_ptr;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;

enum { kFromPool = 0, kFromOwn = 1 };

struct ExtParams {
    const uint16_t* q;
    int64_t q_st, q_sh;
    const uint16_t* kp;            // pool mode: the stripe pools; own mode: the in-step keys and values
    const uint16_t* vp;
    PoolGeom geo;                  // pool mode
    int64_t kv_st, kv_sh;          // own mode: token and head strides of k and v
    const int32_t* row_start;      // q_row_start (pool mode) or cu_seqlens (own mode)
    int32_t* order;                // pool mode with a plan: triples by rank, longest stripe first (null: grid order)
    const int32_t* ctx_len;        // pool mode
    const int32_t* bt;
    int64_t bt_stride;
    float* out;
    int64_t o_ss, o_st, o_sh;
    float* lse;
    int64_t l_ss, l_st;
    int32_t B, T, P, stripe_begin, S, Hq, Hkv, G, max_pages, page_size, max_row_tokens;
    int32_t ctx_cap;        // context lengths are clamped to min(max_pages * page_size, max_ctx_len)
    int32_t n_qblocks, n_units, pad_tokens_per_block;
    int32_t pad_lse_only;   // CPATTN_FLAG_PAD_LSE_ONLY: padding tokens get their lse only
    float scale_log2;       // softmax scale in log2 units (fp8 pools: times the key descale)
    float v_scale;          // fp8 pools: the value descale (1 otherwise)
};

__device__ __forceinline__ int swz(int t) { return (2 * t) & 15; }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to a packed fp16 pair, round to nearest even (inf past the fp16 range).
__device__ __forceinline__ uint32_t pack2_f16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}

// Eight bf16 values to eight fp16 values in the same order: exact for magnitudes in [2^-14, 65504], within 2^-25
// absolute below that.
__device__ __forceinline__ f16x8_t bf16x8_to_f16(u32x4_t v) {
    u32x4_t r;
#pragma unroll
    for (int d = 0; d < 4; ++d) r[d] = pack2_f16(__uint_as_float(v[d] << 16), __uint_as_float(v[d] & 0xffff0000u));
    return __builtin_bit_cast(f16x8_t, r);
}

// s_waitcnt vmcnt(n) with the other counters at their maximum (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without the memory fences of __syncthreads (those would drain the tiles in flight); the empty
// asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Scheduling groups: AHEAD LDS reads first, then (one MFMA, R reads) until the N MFMAs of the region are placed.
template <int N, int R, int AHEAD>
__device__ __forceinline__ void sched_pipeline() {
    constexpr int kDsRead = 0x100, kMfma = 0x008;
    __builtin_amdgcn_sched_group_barrier(kDsRead, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < N - AHEAD / R; ++i) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kDsRead, R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, AHEAD / R, 0);
}

// Element offset (from the K or V base) of key j's row for kv head g (pool mode: the staged page ids are valid ones).
template <int MODE>
__device__ __forceinline__ int64_t key_row(const ExtParams& p, lds_i32_ptr s_pages, int32_t r, int32_t g, int32_t tok0,
                                           int32_t j) {
    if (MODE == kFromPool) {
        const int32_t page = s_pages[j >> p.geo.pp_shift];
        return int64_t(r) * p.geo.s_stripe + int64_t(page) * p.geo.s_page + int64_t(j & (p.geo.pp - 1)) * p.geo.s_slot +
               int64_t(g) * p.geo.s_head;
    } else {
        return int64_t(tok0 + j) * p.kv_st + int64_t(g) * p.kv_sh;
    }
}

// Issue the direct-to-LDS loads of one tile: wave w loads tokens [kTokPerWave w, kTokPerWave (w + 1)) of K and of V,
// four tokens (64 lanes x 16 bytes) an instruction; lane l fills stored piece l % 16 of its token with logical piece
// (l % 16) ^ f(t). Keys past the end take the last key's row (their scores are masked out). fp8 pools: one
// instruction per wave for K and one for V, lane l loading codes [16 (l % 8), +16) of token l / 8, in token order
// into the staging half of the wave's rows.
// One 4-token group i of a bf16 tile, addressed lane by lane.
template <int MODE>
__device__ __forceinline__ void issue_group(const ExtParams& p, lds_i32_ptr s_pages, int32_t r, int32_t g, int32_t tok0,
                                            int32_t tile0, int32_t last_key, lds_char_ptr tile, int32_t w, int lane,
                                            int i) {
    const int32_t t = kTokPerWave * w + 4 * i + (lane >> 4);
    const int64_t off = key_row<MODE>(p, s_pages, r, g, tok0, min(tile0 + t, last_key)) + 8 * ((lane & 15) ^ swz(t));
    const int32_t dst = kRowBytes * (kTokPerWave * w + 4 * i);
    __builtin_amdgcn_global_load_lds((const void*)(p.kp + off), (lds_ptr)(tile + dst), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(p.vp + off), (lds_ptr)(tile + kVOff + dst), 16, 0, 0);
}

template <int MODE, bool KV8>
__device__ __forceinline__ void issue_tile(const ExtParams& p, lds_i32_ptr s_pages, int32_t r, int32_t g, int32_t tok0,
                                           int32_t tile0, int32_t last_key, lds_char_ptr tile, int32_t w, int lane) {
    if constexpr (KV8) {
        const int32_t t = kTokPerWave * w + (lane >> 3);
        const int64_t off = key_row<MODE>(p, s_pages, r, g, tok0, min(tile0 + t, last_key)) + 16 * (lane & 7);
        const int32_t dst = kRowBytes * kTokPerWave * w + kStage8;
        __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(p.kp) + off),
                                         (lds_ptr)(tile + dst), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(p.vp) + off),
                                         (lds_ptr)(tile + kVOff + dst), 16, 0, 0);
        return;
    }
#pragma unroll
    for (int i = 0; i < kTokPerWave / 4; ++i) issue_group<MODE>(p, s_pages, r, g, tok0, tile0, last_key, tile, w, lane, i);
}

// Widen the V rows this wave loaded into a tile (tokens [kTokPerWave w, +kTokPerWave), 256 bytes each, pieces stored
// swizzled) from bf16 to fp16 in place: the value product then reads fp16 operands straight from LDS, and each V
// element is converted once per workgroup instead of once per wave that reads it. Elementwise, so the swizzle of the
// pieces is unchanged.
__device__ __forceinline__ void widen_v_to_f16(lds_char_ptr tile, int32_t w, int lane) {
    constexpr int kBytes = kTokPerWave * kRowBytes;            // this wave's V rows
    static_assert(kBytes % (64 * 16) == 0, "whole 16-byte pieces per lane");
#pragma unroll
    for (int i = 0; i < kBytes / (64 * 16); ++i) {
        __attribute__((address_space(3))) u32x4_t* ptr =
            (__attribute__((address_space(3))) u32x4_t*)(tile + kVOff + kTokPerWave * w * kRowBytes + 16 * (64 * i + lane));
        *ptr = __builtin_bit_cast(u32x4_t, bf16x8_to_f16(*ptr));
    }
}

// Widen the fp8 K and V codes this wave staged into a tile (tokens [kTokPerWave w, +kTokPerWave)) into the layout of
// bf16 tiles: K to bf16, V to fp16, both exact for every E4M3 code. Lane l takes codes [16 j, +16) of token i
// (i = l / 8, j = l % 8), i.e. logical pieces 2j and 2j + 1 of the token's row, which the swizzle (f(t) even) keeps
// adjacent. Each lane's codes are read before any lane writes (one read instruction per tensor, whose results the
// writes wait for), so widening over the staging bytes is safe.
__device__ __forceinline__ void widen_kv_fp8(lds_char_ptr tile, int32_t w, int lane) {
    typedef __attribute__((address_space(3))) u32x4_t* lds_u32x4_ptr;
    const int32_t i = lane >> 3, j = lane & 7;
    const int32_t t = kTokPerWave * w + i;
    const int32_t stage = kRowBytes * kTokPerWave * w + kStage8 + 16 * lane;
    const u32x4_t ck = *(lds_u32x4_ptr)(tile + stage);
    const u32x4_t cv = *(lds_u32x4_ptr)(tile + kVOff + stage);
    u32x4_t k2[2], v2[2];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t kl = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ck[d], 1.0f, false));
        const uint32_t kh = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ck[d], 1.0f, true));
        const uint32_t vl = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cv[d], 1.0f, false));
        const uint32_t vh = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cv[d], 1.0f, true));
        k2[d >> 1][2 * (d & 1)] = kl;
        k2[d >> 1][2 * (d & 1) + 1] = kh;
        v2[d >> 1][2 * (d & 1)] = vl;
        v2[d >> 1][2 * (d & 1) + 1] = vh;
    }
    const int32_t row = kRowBytes * t + 16 * ((2 * j) ^ swz(t));
    *(lds_u32x4_ptr)(tile + row) = k2[0];
    *(lds_u32x4_ptr)(tile + row + 16) = k2[1];
    *(lds_u32x4_ptr)(tile + kVOff + row) = v2[0];
    *(lds_u32x4_ptr)(tile + kVOff + row + 16) = v2[1];
}

// Make a tile this wave loaded ready for the products: V rows to fp16 (bf16 pools) or K and V codes widened (fp8).
template <bool KV8>
__device__ __forceinline__ void widen_tile(lds_char_ptr tile, int32_t w, int lane) {
    if constexpr (KV8)
        widen_kv_fp8(tile, w, lane);
    else
        widen_v_to_f16(tile, w, lane);
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads and writes have completed (the other counters at their maximum).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Maximum of three floats in one instruction. fmaxf would first quiet each operand (IEEE mode), one extra instruction
// per operand; scores and their maxima are never signalling NaNs, so that step is not needed here.
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Reductions over the four 16-lane groups (lanes n, n + 16, n + 32, n + 48) through the gfx950 lane swaps, which stay
// in the vector unit: swapping a register with itself by 32 lanes pairs each lane with its partner in the other half,
// and by 16 lanes within each half.
__device__ __forceinline__ float group_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = max3(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max3(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace

// Plan of the context part: the triples ranked by stripe length, longest first, into p.order. Rows bring very
// different amounts of work (context and in-step lengths both vary), and the hardware hands out workgroups in grid
// order as slots free up: run in row order, the last rows' long units set the end of the launch while most CUs idle.
__global__ __launch_bounds__(256) void gqa_extend_plan_kernel(const ExtParams p) {
    __shared__ __attribute__((aligned(16))) int32_t s_key[kMaxPlanTriples];
    __shared__ int32_t s_part[256];
    const int32_t n = p.n_units / p.Hkv;
    const int32_t npad = rank_padded(n);
    // Key of triple v = (row b, stripe s, query block qb), v = (b S + s) n_qblocks + qb: the stripe length when the
    // block holds query rows, -1 when it lies past the row's rows (such workgroups only return, so they go last).
    const int32_t nq = p.n_qblocks;
    for_each_plan_pair(p.row_start, p.ctx_len, p.B, p.S, p.T, p.max_row_tokens, p.ctx_cap, p.stripe_begin, p.P,
                       p.geo.interleave, [&](int32_t bs, int32_t ntok, int32_t lr) {
                           for (int32_t qb = 0; qb < nq; ++qb) s_key[bs * nq + qb] = qb * kBlockRows < ntok * p.G ? lr : -1;
                       });
    for (int32_t v = n + int32_t(threadIdx.x); v < npad; v += blockDim.x) s_key[v] = -1;
    __syncthreads();
    rank_longest_first(s_key, s_part, n, p.order);
}

// UPAGE (bf16 pools with pages of at least 4 slots): the 4 tokens of a load instruction share one page (the group's
// first key, or the last key for a group past it), read from the staged ids a step ahead; each lane's address is the
// row base plus page times page stride (a 32 x 32 -> 64-bit product) plus its clamped key's slot and its piece. The
// scalar unit, shared by the CU's four SIMDs, is kept out of the 64-bit arithmetic: moved there it became the
// bottleneck.
template <int MODE, bool KV8, bool UPAGE>
__global__ __launch_bounds__(64 * kNW, 2) void gqa_extend_kernel(const ExtParams p) {
    static_assert(MODE == kFromPool || !KV8, "fp8 codes come from the pools only");
    static_assert(!UPAGE || (MODE == kFromPool && !KV8), "uniform pages: bf16 pools");
    constexpr int kLoadsPerTile = loads_per_tile<KV8>();
    // Four tile buffers as separate arrays: a read of one and a tile load into another then refer to different
    // objects, which the wait-count pass needs to see to leave the other tiles' loads in flight.
    __shared__ __attribute__((aligned(16))) char s_tile0[kTileBytes];
    __shared__ __attribute__((aligned(16))) char s_tile1[kTileBytes];
    __shared__ __attribute__((aligned(16))) char s_tile2[kTileBytes];
    __shared__ __attribute__((aligned(16))) char s_tile3[kTileBytes];
    __shared__ int32_t s_pages[kMaxPages];
    const int lane = threadIdx.x & 63;
    const int32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t blk = blockIdx.x;

    if (blk >= p.n_units) {                                 // padding-token fill role
        const int32_t k = blk - p.n_units;
        const int32_t first = min(max(p.row_start[p.B], 0), p.T);
        const int32_t t0 = max(k * p.pad_tokens_per_block, first);
        const int32_t t1 = min((k + 1) * p.pad_tokens_per_block, p.T);
        if (t0 < t1)
            fill_padding(p.out, p.o_ss, p.o_st, p.o_sh, p.lse, p.l_ss, p.l_st, p.S, p.Hq, kD, t0, t1, threadIdx.x,
                         blockDim.x, p.pad_lse_only);
        return;
    }

    // Unit order: kv head fastest, then the (row, stripe, query block) triple: with a plan the triples by rank
    // (longest stripe first; a row's blocks of one stripe stay adjacent), else query block, stripe, row. The hardware
    // hands block i to XCD i mod 8, so with 8 kv heads (or a multiple) every XCD gets one head of every triple: equal
    // work per XCD whatever the mix of row lengths, and the query blocks of one (row, stripe, kv head), which read the
    // same K/V tiles, run on one XCD close together in time and share its L2. In the own-token part a row's query
    // blocks run last block first: a block attends the keys up to its last token, so the long ones start early.
    int32_t v = blk;
    const int32_t g = v % p.Hkv;
    v /= p.Hkv;
    if (MODE == kFromPool && p.order) v = ((const_i32_ptr)p.order)[v];
    if (v < 0) return;                                      // a block past its row's rows (plan key -1)
    const int32_t qb = MODE == kFromOwn ? p.n_qblocks - 1 - v % p.n_qblocks : v % p.n_qblocks;
    v /= p.n_qblocks;
    const int32_t s = v % p.S;
    const int32_t b = v / p.S;
    const const_i32_ptr rs = (const_i32_ptr)p.row_start;
    const int32_t tok0 = min(max(rs[b], 0), p.T);
    const int32_t tok1 = min(max(rs[b + 1], tok0), p.T);
    if (g == 0 && qb == p.n_qblocks - 1)
        fill_excess_tokens(p.out + int64_t(s) * p.o_ss, p.o_st, p.o_sh, p.lse + int64_t(s) * p.l_ss, p.l_st, tok0, tok1,
                           p.max_row_tokens, p.Hq, kD, threadIdx.x, blockDim.x, p.pad_lse_only);
    const int32_t ntok = min(tok1 - tok0, p.max_row_tokens);
    const int32_t nrows = ntok * p.G;
    const int32_t row0 = qb * kBlockRows;
    if (row0 >= nrows) return;
    const int32_t r = p.stripe_begin + s;
    int32_t nkeys;
    if (MODE == kFromPool) {
        const int32_t L = min(max(((const_i32_ptr)p.ctx_len)[b], 0), p.ctx_cap);
        nkeys = stripe_length(L, r, p.P, p.geo.interleave);
    } else {
        nkeys = min(ntok, (min(row0 + kBlockRows, nrows) - 1) / p.G + 1);   // keys up to the block's last token
    }
    const int32_t n16 = lane & 15, c4 = lane >> 4;
    const int32_t wrow0 = row0 + kRowsPerWave * w;          // first query row of this wave
    const bool wave_live = wrow0 < nrows;                   // wave-uniform

    if (nkeys == 0) {                                       // no key: (0, -inf) for this wave's rows
        if (wave_live) {
            for (int32_t rr = 0; rr < kRowsPerWave; ++rr) {
                const int32_t rho = wrow0 + rr;
                if (rho >= nrows) break;
                const int32_t t = tok0 + rho / p.G, h = g * p.G + rho % p.G;
                float* o = p.out + int64_t(s) * p.o_ss + int64_t(t) * p.o_st + int64_t(h) * p.o_sh;
                for (int32_t d = lane; d < kD; d += 64) o[d] = 0.f;
                if (lane == 0) p.lse[int64_t(s) * p.l_ss + int64_t(t) * p.l_st + h] = neg_inf();
            }
        }
        return;
    }
    const int32_t ntiles = (nkeys + kTile - 1) / kTile;
    const int32_t last_key = nkeys - 1;

    // Query operand: rows wrow0 + 16 rb + n16, dims [32 ks + 8 c4, +8); rows past the end read zeros.
    u32x4_t qreg[2][4];
    int32_t qtok[2];                                        // the row's token within the row (for the causal mask)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int32_t rho = wrow0 + 16 * rb + n16;
        qtok[rb] = rho / p.G;
        if (rho < nrows) {
            const uint16_t* qp = p.q + int64_t(tok0 + rho / p.G) * p.q_st + int64_t(g * p.G + rho % p.G) * p.q_sh + 8 * c4;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qreg[rb][ks] = *reinterpret_cast<const u32x4_t*>(qp + 32 * ks);
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qreg[rb][ks] = (u32x4_t){0u, 0u, 0u, 0u};
        }
    }

    // The stripe's page ids, staged once in LDS (at most kMaxPages by the eligibility check). The barrier's wait also
    // retires the query loads above, so nothing but tile loads is outstanding inside the loop.
    if (MODE == kFromPool) {
        const int32_t npages = (last_key >> p.geo.pp_shift) + 1;
        const int32_t* bt_row = p.bt + int64_t(b) * p.bt_stride;
        for (int32_t i = threadIdx.x; i < npages; i += blockDim.x) {
            const int32_t pg = bt_row[i];
            s_pages[i] = (pg >= 0 && pg < p.geo.num_pages) ? pg : 0;   // ids outside the pool read page 0
        }
    }
    __syncthreads();
    const lds_i32_ptr pages = (lds_i32_ptr)s_pages;

    // Per-lane LDS byte offsets inside a tile (reads add the buffer address as an immediate):
    //   score operand: token 16 tb + n16, logical piece 4 ks + c4;
    //   value operand through transposed reads: in each 16-lane group, lane s supplies four consecutive values of one
    //   row and lane q receives element q % 4 of rows q / 4, 4 + q / 4, 8 + q / 4, 12 + q / 4. Lane s of group c4
    //   points at token 16 rr + 4 c4 + s / 4, dims 16 db + 4 (s % 4), so lane q receives dim 16 db + q of tokens
    //   8 c4 + e in k order: the B operand of dim block db.
    int32_t kofs[2][4], vofs[2][8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int32_t t = 16 * tb + n16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kofs[tb][ks] = kRowBytes * t + 16 * ((4 * ks + c4) ^ swz(t));
    }
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int32_t t = 16 * rr + 4 * c4 + (n16 >> 2);
#pragma unroll
        for (int db = 0; db < 8; ++db)
            vofs[rr][db] = kVOff + kRowBytes * t + 16 * ((2 * db + ((n16 >> 1) & 1)) ^ swz(t)) + 8 * (n16 & 1);
    }

    // Uniform-page addressing: the row base of (stripe, kv head) and each lane's stored-piece offset, the same on
    // every tile; V rows lie a fixed distance from K rows.
    const uint64_t kbase =
        reinterpret_cast<uint64_t>(p.kp + int64_t(r) * p.geo.s_stripe + int64_t(g) * p.geo.s_head);
    const int64_t v_minus_k = (reinterpret_cast<const char*>(p.vp) - reinterpret_cast<const char*>(p.kp));
    const uint32_t page_bytes = uint32_t(2 * p.geo.s_page);       // below 2^32 (launch condition)
    const uint32_t slot_bytes = uint32_t(2 * p.geo.s_slot);       // slot_bytes * pp below 2^31 (launch condition)
    uint32_t piece_off[kTokPerWave / 4];
#pragma unroll
    for (int i = 0; i < kTokPerWave / 4; ++i)
        piece_off[i] = uint32_t(16 * ((lane & 15) ^ swz(kTokPerWave * w + 4 * i + (lane >> 4))));
    // Page ids of this wave's groups of the tile starting at key tile0 (uniform pages only).
    auto tile_pages = [&](int32_t tile0, int32_t (&pg)[kTokPerWave / 4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kTokPerWave / 4; ++i)
            pg[i] = UPAGE ? pages[min(tile0 + kTokPerWave * w + 4 * i, last_key) >> p.geo.pp_shift] : 0;
    };
    auto issue = [&](int32_t tile0, lds_char_ptr tile, const int32_t (&pg)[kTokPerWave / 4])
        __attribute__((always_inline)) {
        if constexpr (UPAGE) {
#pragma unroll
            for (int i = 0; i < kTokPerWave / 4; ++i) {
                // the lane's key, clamped to the last one: on the group's page (pg[i]) whichever way it is clamped
                const int32_t j = min(tile0 + kTokPerWave * w + 4 * i + (lane >> 4), last_key);
                const uint64_t ka = uint64_t(uint32_t(pg[i])) * page_bytes + kbase +
                                    (uint32_t(j & (p.geo.pp - 1)) * slot_bytes + piece_off[i]);
                const int32_t dst = kRowBytes * (kTokPerWave * w + 4 * i);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(ka), (lds_ptr)(tile + dst), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(ka + v_minus_k),
                                                 (lds_ptr)(tile + kVOff + dst), 16, 0, 0);
            }
        } else {
            issue_tile<MODE, KV8>(p, pages, r, g, tok0, tile0, last_key, tile, w, lane);
        }
    };

    auto tile_buf = [&](auto bc) __attribute__((always_inline)) -> lds_char_ptr {
        constexpr int bb = decltype(bc)::value % kBufs;
        return bb == 0 ? (lds_char_ptr)s_tile0 : bb == 1 ? (lds_char_ptr)s_tile1 : bb == 2 ? (lds_char_ptr)s_tile2
                                                                                     : (lds_char_ptr)s_tile3;
    };
    f32x4_t o[2][8];                                        // o[rb][db][i]: row 16 rb + 4 c4 + i, dim 16 db + n16
    // m: softmax reference of each row in raw score units (p = 2^((s - m) * scale_log2)); l: the rows' sums of p (for
    // the lse); lr: the rows' sums of the fp16-rounded p that weight the values (for the normalisation).
    float m[2], l[2], lr[2];
    auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int db = 0; db < 8; ++db) o[rb][db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            m[rb] = neg_inf();
            l[rb] = 0.f;
            lr[rb] = 0.f;
        }
    };

    // kAhead tiles in flight before the loop; every iteration issues one more (tile indices past the end re-read the
    // last tile into a buffer nobody reads), so the wait at the top of an iteration leaves exactly the kAhead - 1
    // newest tiles' loads (kLoadsPerTile instructions each) outstanding.
    //
    // The prologue's loads take their LDS address through an opaque copy of the buffer pointer. The compiler's
    // wait-count pass then does not track them against the buffer arrays; tracked, their state merged into the loop
    // header's and made it wait for every load in flight there (a full drain every fourth tile). The explicit wait
    // and barrier at the top of each step order these loads before the reads of their tiles all the same.
    auto opaque = [](lds_char_ptr t) __attribute__((always_inline)) {
        asm volatile("" : "+v"(t));
        return t;
    };
    auto prologue = [&]() __attribute__((always_inline)) {
        int32_t pg[kTokPerWave / 4];
        tile_pages(0, pg);
        issue(0, opaque(tile_buf(std::integral_constant<int, 0>{})), pg);
        tile_pages(min(kTile, (ntiles - 1) * kTile), pg);
        issue(min(kTile, (ntiles - 1) * kTile), opaque(tile_buf(std::integral_constant<int, 1>{})), pg);
        tile_pages(min(2 * kTile, (ntiles - 1) * kTile), pg);
        issue(min(2 * kTile, (ntiles - 1) * kTile), opaque(tile_buf(std::integral_constant<int, 2>{})), pg);
        wait_vmcnt<(kAhead - 1) * kLoadsPerTile>();         // this wave's pieces of tile 0 are in LDS
        asm volatile("" ::: "memory");                      // (the LDS reads below stay after the wait)
        widen_tile<KV8>(opaque(tile_buf(std::integral_constant<int, 0>{})), w, lane);
        wait_lgkm0();
    };
    static_assert(kAhead == 3 && kBufs == 4, "ring");

    // Raw scores of tile kt for this wave's rows, sv[rb][e] = S[row 16 rb + n16][key 16 (e / 4) + 4 c4 + e % 4], with
    // keys past the end and (own-token part) keys after the row's token set to -inf.
    auto tile_scores = [&](lds_char_ptr tile, int32_t kt, float (&sv)[2][8]) __attribute__((always_inline)) {
        const int32_t tile0 = kt * kTile;
        // Masking is needed on the last tile and, for the own-token part, on tiles reaching past this wave's first
        // query token (wave-uniform conditions).
        const bool mask = tile0 + kTile > nkeys || (MODE == kFromOwn && tile0 + kTile - 1 > wrow0 / p.G);
        f32x4_t sacc[2][2];                                 // S^T[key 16 tb + 4 c4 + i][row 16 rb + n16]
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) sacc[rb][tb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const u32x4_t kv = *(const __attribute__((address_space(3))) u32x4_t*)(tile + kofs[tb][ks]);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    sacc[rb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), as_bf16x8(qreg[rb][ks]),
                                                                           sacc[rb][tb], 0, 0, 0);
            }
        }
        sched_pipeline<16, 1, 4>();
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[rb][e] = sacc[rb][e >> 2][e & 3];
            if (mask) {
                // key j = tile0 + off + 4 c4 with off = 16 (e / 4) + e % 4: the lane's part 4 c4 is compared with
                // wave-uniform bounds, so unmasked tiles carry no per-key index arithmetic
                const int32_t kleft = nkeys - tile0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int32_t off = 16 * (e >> 2) + (e & 3);
                    if (4 * c4 >= kleft - off || (MODE == kFromOwn && 4 * c4 - qtok[rb] > -(tile0 + off)))
                        sv[rb][e] = neg_inf();
                }
            }
        }
    };
    auto row_max = [&](const float (&sv)[8]) __attribute__((always_inline)) {
        return group_max(max3(max3(sv[0], sv[1], sv[2]), max3(sv[3], sv[4], sv[5]), max3(sv[6], sv[7], sv[7])));
    };

    // One tile: scores, probabilities relative to the row references m, out += P . V.
    auto tile_compute = [&](lds_char_ptr tile, int32_t kt) __attribute__((always_inline)) {
        float sv[2][8];
        tile_scores(tile, kt, sv);
        const float c = p.scale_log2;
        // p = 2^((s - m) * scale_log2): one fused multiply-add per score (the launch requires scale_log2 > 0, which
        // keeps the order of the scores); P enters the value product rounded to fp16 (11 significant bits).
        u32x4_t ph[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const float mc = -m[rb] * c;
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[rb][e], c, mc));
            l[rb] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
#pragma unroll
            for (int d = 0; d < 4; ++d) ph[rb][d] = pack2_f16(pv[2 * d], pv[2 * d + 1]);
            typedef __fp16 h2_t __attribute__((ext_vector_type(2)));
            const h2_t one2 = __builtin_bit_cast(h2_t, 0x3c003c00u);       // (1.0, 1.0)
            float lsum = 0.f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t pd = ph[rb][d];
                lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, pd), one2, lsum, false);
            }
            lr[rb] += lsum;
        }

        // Values: 8 output tiles of 16 dims per row block, each B operand from two transposed reads, widened from bf16
        // to fp16 in registers. The wave issues them at raised priority: with two waves a SIMD, the other wave's
        // softmax then fills the gaps between these MFMAs instead of delaying them (measured 0.8% faster on bf16 pools,
        // 1.5% on fp8 pools).
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(tile + vofs[0][db]));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(tile + vofs[1][db]));
            const f16x8_t bop =
                __builtin_bit_cast(f16x8_t, (s16x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, ph[rb]), bop, o[rb][db],
                                                                  0, 0, 0);
        }
        sched_pipeline<16, 1, 8>();
        __builtin_amdgcn_s_setprio(0);
    };

    // One iteration with buffer bb (compile time): wait for tile kt, issue the loads of tile kt + kAhead into buffer
    // bb + kAhead, compute tile kt from buffer bb.
    // Waves past the last query row still load their share of every tile; they run the same loop (same barriers)
    // without the compute, as a separate copy so that no branch on liveness sits inside the pipelined loop.
    auto step = [&](auto bc, auto live, auto maxonly, int32_t kt) __attribute__((always_inline)) {
        constexpr int bb = decltype(bc)::value;
        // The page ids of the tile issued below are read first; the wait for this step's LDS work covers them.
        const int32_t tnext = min((kt + kAhead) * kTile, (ntiles - 1) * kTile);
        int32_t pg[kTokPerWave / 4];
        tile_pages(tnext, pg);
        // This wave's pieces of tiles kt and kt + 1 are in LDS (tile kt already widened by every wave before the
        // barrier below; tile kt + 1 is widened at the end of this step, before the next step's barrier: after the
        // compute, measured 2.5% faster than before it).
        wait_vmcnt<(kAhead - 2) * kLoadsPerTile>();
        wait_lgkm0();
        lds_barrier();                                      // every wave's too; tile kt - 1's buffer is free
        issue(tnext, tile_buf(std::integral_constant<int, bb + kAhead>{}), pg);
        if constexpr (decltype(live)::value) {
            if constexpr (decltype(maxonly)::value) {
                float sv[2][8];
                tile_scores(tile_buf(std::integral_constant<int, bb>{}), kt, sv);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) m[rb] = fmaxf(m[rb], row_max(sv[rb]));
            } else {
                tile_compute(tile_buf(std::integral_constant<int, bb>{}), kt);
            }
        }
        widen_tile<KV8>(tile_buf(std::integral_constant<int, bb + 1>{}), w, lane);
    };
    auto run = [&](auto live, auto maxonly) __attribute__((always_inline)) {
        for (int32_t kt = 0; kt < ntiles; kt += kBufs) {
            step(std::integral_constant<int, 0>{}, live, maxonly, kt);
            if (kt + 1 >= ntiles) break;
            step(std::integral_constant<int, 1>{}, live, maxonly, kt + 1);
            if (kt + 2 >= ntiles) break;
            step(std::integral_constant<int, 2>{}, live, maxonly, kt + 2);
            if (kt + 3 >= ntiles) break;
            step(std::integral_constant<int, 3>{}, live, maxonly, kt + 3);
        }
        wait_vmcnt<0>();                                    // the over-issued tail loads land
    };

    // Epilogue: row sums over the four lane groups, then the normalised rows and their lse. Returns true when a sum or
    // an accumulator is inf or NaN.
    auto store = [&]() __attribute__((always_inline)) -> bool {
        float z = 0.f;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float ls = l[rb];
            ls = group_sum(ls);
            const float lrs = group_sum(lr[rb]);
            z += 0.f * ls;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t rho = wrow0 + 16 * rb + 4 * c4 + i;
                const float li = __shfl(lrs, 4 * c4 + i);
#pragma unroll
                for (int db = 0; db < 8; ++db) z += 0.f * o[rb][db][i];
                if (rho < nrows) {
                    const float inv = li > 0.f ? (KV8 ? p.v_scale : 1.0f) / li : 0.f;
                    const int32_t t = tok0 + rho / p.G, h = g * p.G + rho % p.G;
                    float* dst = p.out + int64_t(s) * p.o_ss + int64_t(t) * p.o_st + int64_t(h) * p.o_sh + n16;
#pragma unroll
                    for (int db = 0; db < 8; ++db) dst[16 * db] = o[rb][db][i] * inv;
                }
            }
            const int32_t rho = wrow0 + 16 * rb + n16;
            if (c4 == 0 && rho < nrows) {
                const int32_t t = tok0 + rho / p.G, h = g * p.G + rho % p.G;
                p.lse[int64_t(s) * p.l_ss + int64_t(t) * p.l_st + h] =
                    ls > 0.f ? (m[rb] * p.scale_log2 + log2f(ls)) * kLn2 : neg_inf();
            }
        }
        return !(z == 0.f);
    };

    // The reference m of each row is the maximum of its first tile's scores (key 0 is valid for every row, so it is
    // finite), and the loop never moves it. A later score above the reference by more than about 16 (log2 units)
    // overflows the fp16 weights (and further on p and the sums) to inf; the workgroup then finds the exact row maxima with a
    // scores-only pass and runs the loop once more (every p now at most 1), overwriting the rows it stored. Any other
    // outcome is the same softmax with a different reference.
    reset();
    prologue();
    lds_barrier();
    if (wave_live) {
        float sv[2][8];
        tile_scores(tile_buf(std::integral_constant<int, 0>{}), 0, sv);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) m[rb] = row_max(sv[rb]);
    }
    for (int32_t attempt = 0;; ++attempt) {
        if (wave_live)
            run(std::true_type{}, std::false_type{});
        else
            run(std::false_type{}, std::false_type{});
        const bool bad = wave_live && store();
        if (attempt > 0 || !__syncthreads_or(bad)) return;
        reset();
        prologue();
        if (wave_live)
            run(std::true_type{}, std::true_type{});
        else
            run(std::false_type{}, std::true_type{});
        prologue();
    }
}

// ------------------------------------------------------------------------------------------------------------ host
namespace {

bool al16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

int32_t launch_extend(ExtParams& p, int mode, bool kv8, hipStream_t stream) {
    const int64_t rows = int64_t(std::max(1, p.max_row_tokens)) * p.G;
    p.n_qblocks = int32_t((rows + kBlockRows - 1) / kBlockRows);
    const int64_t units = int64_t(p.B) * p.S * p.Hkv * p.n_qblocks;
    p.n_units = int32_t(units);
    p.pad_tokens_per_block = 4;
    const int64_t blocks = units + (p.T + 3) / 4;
    if (blocks == 0) return CPATTN_OK;
    if (p.order && units > 0) {
        hipLaunchKernelGGL(gqa_extend_plan_kernel, dim3(uint32_t((units / p.Hkv + kRankItems - 1) / kRankItems)), dim3(256),
                           0, stream, p);
        if (int32_t st = check_launch("cp_paged_attn_partial (extend plan)")) return st;
    }
    const dim3 grid{uint32_t(blocks), 1, 1};
    if (mode == kFromPool && kv8)
        hipLaunchKernelGGL((gqa_extend_kernel<kFromPool, true, false>), grid, dim3(64 * kNW), 0, stream, p);
    else if (mode == kFromPool && p.geo.pp_shift >= 2 && 2 * p.geo.s_page < (int64_t(1) << 32) &&
             2 * p.geo.s_slot * p.geo.pp < (int64_t(1) << 31))
        hipLaunchKernelGGL((gqa_extend_kernel<kFromPool, false, true>), grid, dim3(64 * kNW), 0, stream, p);
    else if (mode == kFromPool)
        hipLaunchKernelGGL((gqa_extend_kernel<kFromPool, false, false>), grid, dim3(64 * kNW), 0, stream, p);
    else
        hipLaunchKernelGGL((gqa_extend_kernel<kFromOwn, false, false>), grid, dim3(64 * kNW), 0, stream, p);
    return check_launch(mode == kFromPool ? "cp_paged_attn_partial (bf16 extend)" : "cp_own_token_attn (bf16)");
}

}  // namespace

bool extend_bf16_eligible(const cp_paged_args& a, const PoolGeom& geo) {
    if (a.kind != CPATTN_GQA || a.dtype != CPATTN_BF16 || a.head_dim != kD || a.head_dim_v != kD) return false;
    const bool kv8 = a.kv_format == CPATTN_KV_FP8_E4M3;
    if (a.kv_format != CPATTN_KV_SAME && !kv8) return false;
    // The softmax tracks the maximum of unscaled scores, so the scale (times the key descale) must be positive.
    if (!(a.scale > 0.f && a.scale < INFINITY)) return false;
    if (kv8 && !(a.scale * a.k_descale > 0.f && a.scale * a.k_descale < INFINITY)) return false;
    const int32_t G = a.num_q_heads / a.num_kv_heads;
    if (kBlockRows % G != 0) return false;
    if (int64_t(a.max_row_tokens) * G <= 16) return false;   // decode-shaped: the decode kernel serves it
    if (geo.pp_shift < 0) return false;
    const int64_t max_lr = max_stripe_length(a);
    if ((max_lr + geo.pp - 1) / geo.pp > kMaxPages) return false;
    if (!al16(a.q) || !al16(a.k_pool) || !al16(a.v_pool)) return false;
    if ((a.q_stride_token | a.q_stride_head) & 7) return false;
    // 16-byte pieces of every pool row: 8 bf16 elements or 16 fp8 codes
    if ((a.kv_stride_stripe | a.kv_stride_page | a.kv_stride_slot | a.kv_stride_head) & (kv8 ? 15 : 7)) return false;
    if (int64_t(a.num_rows) * a.stripe_count * a.num_kv_heads * ((int64_t(a.max_row_tokens) * G + kBlockRows - 1) /
                                                                  kBlockRows) + (a.num_tokens + 3) / 4 >
        (int64_t(1) << 31) - 1)
        return false;
    return true;
}

// (row, stripe, query block) triples of a context-part launch, and the workspace of its plan: one int32 rank entry a
// triple, when there are at least two and at most kMaxPlanTriples (otherwise the units run in grid order).
int64_t extend_triples(const cp_paged_args& a) {
    const int64_t G = a.num_q_heads / a.num_kv_heads;
    return int64_t(a.num_rows) * a.stripe_count * ((int64_t(std::max(1, a.max_row_tokens)) * G + kBlockRows - 1) / kBlockRows);
}

int64_t extend_bf16_workspace_bytes(const cp_paged_args& a) {
    const int64_t n = extend_triples(a);
    return n >= 2 && n <= kMaxPlanTriples ? (4 * n + 255) / 256 * 256 : 0;
}

int32_t launch_paged_extend_bf16(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream) {
    ExtParams p{};
    p.order = extend_bf16_workspace_bytes(a) > 0 ? static_cast<int32_t*>(a.workspace) : nullptr;
    p.q = static_cast<const uint16_t*>(a.q);
    p.q_st = a.q_stride_token;
    p.q_sh = a.q_stride_head;
    p.kp = static_cast<const uint16_t*>(a.k_pool);
    p.vp = static_cast<const uint16_t*>(a.v_pool);
    p.geo = geo;
    p.row_start = a.q_row_start;
    p.ctx_len = a.ctx_len;
    p.bt = a.block_table;
    p.bt_stride = a.bt_stride;
    p.out = a.out;
    p.o_ss = a.out_stride_stripe;
    p.o_st = a.out_stride_token;
    p.o_sh = a.out_stride_head;
    p.lse = a.lse;
    p.l_ss = a.lse_stride_stripe;
    p.l_st = a.lse_stride_token;
    p.B = a.num_rows;
    p.T = a.num_tokens;
    p.P = a.num_partners;
    p.stripe_begin = a.stripe_begin;
    p.S = a.stripe_count;
    p.Hq = a.num_q_heads;
    p.Hkv = a.num_kv_heads;
    p.G = a.num_q_heads / a.num_kv_heads;
    p.max_pages = a.max_pages;
    p.ctx_cap = ctx_cap_of(a);
    p.page_size = a.page_size;
    p.max_row_tokens = a.max_row_tokens;
    const bool kv8 = a.kv_format == CPATTN_KV_FP8_E4M3;
    p.scale_log2 = a.scale * (kv8 ? a.k_descale : 1.0f) * kLog2e;
    p.v_scale = kv8 ? a.v_descale : 1.0f;
    p.pad_lse_only = (a.flags & CPATTN_FLAG_PAD_LSE_ONLY) ? 1 : 0;
    return launch_extend(p, kFromPool, kv8, stream);
}

bool own_bf16_eligible(const cp_own_args& a) {
    if (a.dtype != CPATTN_BF16 || a.head_dim != kD) return false;
    if (!(a.scale > 0.f && a.scale < INFINITY)) return false;
    const int32_t G = a.num_q_heads / a.num_kv_heads;
    if (kBlockRows % G != 0) return false;
    if (!al16(a.q) || !al16(a.k) || !al16(a.v)) return false;
    if ((a.q_stride_token | a.q_stride_head | a.kv_stride_token | a.kv_stride_head) & 7) return false;
    if (int64_t(a.num_rows) * a.num_kv_heads * ((int64_t(std::max(1, a.max_row_tokens)) * G + kBlockRows - 1) /
                                                 kBlockRows) + (a.bucket_tokens + 3) / 4 >
        (int64_t(1) << 31) - 1)
        return false;
    return true;
}

int32_t launch_own_token_bf16(const cp_own_args& a, hipStream_t stream) {
    ExtParams p{};
    p.q = static_cast<const uint16_t*>(a.q);
    p.q_st = a.q_stride_token;
    p.q_sh = a.q_stride_head;
    p.kp = static_cast<const uint16_t*>(a.k);
    p.vp = static_cast<const uint16_t*>(a.v);
    p.kv_st = a.kv_stride_token;
    p.kv_sh = a.kv_stride_head;
    p.row_start = a.cu_seqlens;
    p.out = a.out;
    p.o_ss = 0;
    p.o_st = a.out_stride_token;
    p.o_sh = a.out_stride_head;
    p.lse = a.lse;
    p.l_ss = 0;
    p.l_st = a.lse_stride_token;
    p.B = a.num_rows;
    p.T = a.bucket_tokens;
    p.P = 1;
    p.S = 1;
    p.Hq = a.num_q_heads;
    p.Hkv = a.num_kv_heads;
    p.G = a.num_q_heads / a.num_kv_heads;
    p.max_pages = 0;
    p.page_size = 1;
    p.max_row_tokens = a.max_row_tokens;
    p.scale_log2 = a.scale * kLog2e;
    p.v_scale = 1.0f;
    p.pad_lse_only = (a.flags & CPATTN_FLAG_PAD_LSE_ONLY) ? 1 : 0;
    return launch_extend(p, kFromOwn, false, stream);
}

}  // namespace cpattn
