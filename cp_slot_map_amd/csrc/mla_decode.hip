// MLA per-stripe paged partial over bf16 or fp8 E4M3 latent pools (one latent head: key = the 576-value latent row,
// value = its first 512 values), built for gfx950 MFMA.
//
// What it computes is the partial of one partner over the slots it holds, returned as (out, natural-log lse), with the
// one latent head of MLA shared by all query heads (mstar PR #1124, "Context / Sequence Parallel 1/5", PR description:
// the context-parallel decode covers MLA's single latent head as well as GQA).
//
// Work decomposition. A unit is (row b, stripe s, query token, chunk of the stripe's local tokens). One workgroup of
// NW = Hq / 16 waves (eight for 128 heads, two per SIMD) serves all query heads of a unit, so each latent tile is
// fetched once. The latent rows stream through LDS in tiles of 32 tokens (four buffers, three tiles in flight), loaded
// straight from global memory into LDS. The two products split the work differently:
//   * scores: wave w owns query heads [16 w, 16 w + 16) (their query operand, 72 VGPRs, stays in registers) and reads
//     the whole key tile;
//   * output: wave w owns value dims [512 w / NW, 512 (w + 1) / NW) of every head (128 accumulator VGPRs) and reads
//     only its slice of the value tile. The probabilities of all heads go through a 1 KB-per-wave LDS buffer.
// Reading the whole value tile in every wave (the other split of the output product) cost 32 KB of transposing LDS
// reads per wave and tile, more than the key reads; with the slice it is 4 KB of value plus 8 KB of probabilities.
// The chunk's page ids are staged in LDS when a unit starts. A small plan kernel orders the units longest first, so
// the hardware's in-order dispatch packs long and short units onto the same compute unit. A stripe longer than one
// chunk leaves one unnormalised record per chunk and a merge kernel combines them exactly.
//
// Per tile and wave (16 heads x 32 tokens):
//   * scores S^T[token][head] = K . Q^T with v_mfma_f32_16x16x32_bf16: A = latent rows (token per lane, 8 dims per
//     lane group), B = the wave's query heads, held in registers for the whole unit. 36 MFMAs.
//   * softmax in log2 units against a fixed per-head reference, the maximum of the unit's first tile; later scores
//     may exceed it by up to 15 without rescaling anything (p <= 2^15 stays inside the fp16 range; a unit whose
//     scores rise further is repeated with the exact maximum as reference). The accumulators are thus written only by
//     MFMAs and stay in the accumulation registers. The running sum adds the fp32 probabilities, so the lse keeps fp32
//     accuracy.
//   * the value product weights by the probabilities rounded to fp16 (11 significant bits) and the output is
//     normalised by the sum of exactly those rounded weights, so the applied weights sum to one. One bf16 rounding
//     (8 bits) put a two-token stripe 2.5e-3 away from the float64 result; with fp16 weights the error bound is
//     eight times smaller, at the cost of widening each value operand from bf16 to fp16 in registers (exact for the
//     latent's magnitudes: values must stay below 65504 in magnitude).
//   * the probabilities (fp16) go to the wave's slot of the LDS probability buffer in the A-operand layout the score
//     product leaves (k index 8c + e of lane group c is tile token 16 (e / 4) + 4c + e % 4); one barrier.
//   * out += P . V with v_mfma_f32_16x16x32_f16 over the wave's 32 / NW dim blocks and the NW head groups: A = a head
//     group's probabilities (one 16-byte LDS read per lane), B = a 16-dim value block from two transposed LDS reads
//     (ds_read_b64_tr_b16) in the same k order, widened to fp16, so no register staging or permutes are needed. 32
//     MFMAs into 128 accumulator registers.
//
// LDS layout of a tile (37,888 bytes; four buffers): the value dims [0, 512) of token t in a row of 1056 bytes at
// 1056 t (1024 bytes of data, 32 of padding), the rope dims [512, 576) in a 128-byte row at 33,792 + 128 t whose eight
// 16-byte pieces are stored XOR g(t) = (t ^ (t >> 2)) & 7. Measured on gfx950, the three read patterns (sixteen
// tokens at one 16-byte piece for the score operand, in either region, and the transposed reads of four tokens for
// the value operand) then run at the full rate of their instruction; with unpadded 1024-byte rows they run at an
// eighth of it.
#include "launch.h"

#include <type_traits>

namespace cpattn {

namespace {

constexpr int kD = 576;                        // latent row (key) length
constexpr int kDv = 512;                       // value length
constexpr int kTile = 32;                      // tokens per LDS tile
constexpr int kRowV = 1056;                    // LDS bytes per token for dims [0, 512): 1024 + 32 of padding
constexpr int kRegionV = kTile * kRowV;        // value-dim region of a tile
constexpr int kRowR = 128;                     // LDS bytes per token for the rope dims [512, 576)
constexpr int kTileBytes = kRegionV + kTile * kRowR;
constexpr int kBufs = 4;                       // LDS tile buffers: three tiles in flight while one is computed
constexpr int kAhead = kBufs - 1;
constexpr int kMaxChunkPages = 512;            // page ids of one chunk staged in LDS
constexpr int kKSteps = kD / 32;               // k-steps of the score product
constexpr int kMaxPlanUnits = 1024;            // units sorted by the plan kernel (block order above)
constexpr int kTargetUnits = 512;              // about two units per compute unit before chunks are split
constexpr int kFp8Off = kRowV - 1024;          // fp8 tiles: a token's 576 codes land at [kFp8Off, kFp8Off + 576) of its row

typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;
typedef __attribute__((address_space(3))) char* lds_char_ptr;
typedef const __attribute__((address_space(3))) int32_t* lds_i32_ptr;

struct MlaParams {
    const uint16_t* q;
    int64_t q_st, q_sh;
    const char* kv;         // latent pool (bytes): bf16 rows, or fp8 E4M3 codes
    PoolGeom geo;
    const int32_t* q_row_start;
    const int32_t* ctx_len;
    const int32_t* bt;
    int64_t bt_stride;
    float* out;
    int64_t o_ss, o_st, o_sh;
    float* lse;
    int64_t l_ss, l_st;
    float* ws_rec;          // n_units records of rec_floats when n_chunks > 1
    int32_t* order;         // unit of each block, longest first; null: block order
    int32_t* ws_redo;       // per workgroup of the first launch: 1 when its scores outgrew their reference
    float* ws_max;          // per (unit, query head): exact score maximum (log2 units) of a unit to redo
    int64_t rec_floats;
    int32_t B, T, P, stripe_begin, S, Hq, max_pages, page_size, max_row_tokens;
    int32_t unit_tokens;   // query tokens per (row, stripe) in the unit space: max(1, max_row_tokens)
    int32_t ctx_cap;        // context lengths are clamped to min(max_pages * page_size, max_ctx_len)
    int32_t n_chunks, chunk_tokens, n_units, pad_blocks, pad_tokens_per_block;
    int32_t head_groups, work_blocks;   // workgroups per unit (1 or 2) and blocks before the padding role
    int32_t pad_lse_only;   // CPATTN_FLAG_PAD_LSE_ONLY: padding tokens get their lse only
    float scale_log2;       // softmax scale (times the latent descale for fp8 pools) in log2 units
    float v_scale;          // latent descale of fp8 pools (applied to the output), else 1
};

__device__ __forceinline__ int swz(int t) { return (t ^ (t >> 2)) & 7; }   // rope-region piece swizzle

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to a packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack2_f16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}

// Eight bf16 values (packed pairs) to eight fp16 values in the same order: exact for magnitudes in [2^-14, 65504],
// within 2^-25 absolute below that.
__device__ __forceinline__ f16x8_t bf16x8_to_f16(u32x4_t v) {
    u32x4_t r;
#pragma unroll
    for (int d = 0; d < 4; ++d) r[d] = pack2_f16(__uint_as_float(v[d] << 16), __uint_as_float(v[d] & 0xffff0000u));
    return __builtin_bit_cast(f16x8_t, r);
}

struct Unit {
    int32_t b, s, qtok, c;
    int32_t t;           // query token (bucket index)
    int32_t Lr;          // stripe length
    int32_t j0, j1;      // chunk range of local tokens
    int32_t tok0, tok1;  // the row's tokens in the bucket
    bool live;           // the row has this query token
};

__device__ __forceinline__ Unit decode_unit(const MlaParams& p, int32_t u) {
    const const_i32_ptr qrs = (const_i32_ptr)p.q_row_start;
    const const_i32_ptr cl = (const_i32_ptr)p.ctx_len;
    Unit x;
    x.c = u % p.n_chunks;
    int32_t v = u / p.n_chunks;
    x.qtok = v % p.unit_tokens;
    v /= p.unit_tokens;
    x.s = v % p.S;
    x.b = v / p.S;
    const int32_t tok0 = min(max(qrs[x.b], 0), p.T);
    const int32_t tok1 = min(max(qrs[x.b + 1], tok0), p.T);
    const int32_t ntok = min(tok1 - tok0, p.max_row_tokens);
    x.live = x.qtok < ntok;
    x.t = tok0 + x.qtok;
    x.tok0 = tok0;
    x.tok1 = tok1;
    const int32_t L = min(max(cl[x.b], 0), p.ctx_cap);
    x.Lr = stripe_length(L, p.stripe_begin + x.s, p.P, p.geo.interleave);
    x.j0 = x.c * p.chunk_tokens;
    x.j1 = min(x.j0 + p.chunk_tokens, x.Lr);
    return x;
}

// Byte address of tile token L % 32's latent row in lane L, from the chunk's page ids staged in LDS (tokens past the
// chunk end take its last token, whose values are masked out; invalid page ids read page 0).
template <bool KV8>
__device__ __forceinline__ uint64_t token_rows(const MlaParams& p, lds_i32_ptr s_pages, int32_t pidx0, int32_t tile0,
                                               int32_t j_last, const char* kv_r, int lane) {
    const int32_t j = min(tile0 + (lane & 31), j_last);
    int32_t page = s_pages[(j >> p.geo.pp_shift) - pidx0];
    page = (page >= 0 && page < p.geo.num_pages) ? page : 0;
    const int64_t row = int64_t(page) * p.geo.s_page + int64_t(j & (p.geo.pp - 1)) * p.geo.s_slot;   // elements
    return reinterpret_cast<uint64_t>(kv_r) + (uint64_t(row) << (KV8 ? 0 : 1));
}

// Cache policy of the latent loads: nontemporal (CPATTN_MLA_NONTEMPORAL, default on), as every latent row is read
// once per call.
#ifndef CPATTN_MLA_NONTEMPORAL
#define CPATTN_MLA_NONTEMPORAL 1
#endif
constexpr int kLatentCpol = CPATTN_MLA_NONTEMPORAL ? 2 : 0;     // 2: the nt bit of the load's cache-policy field

// Issue the direct-to-LDS loads of one tile.
//   * value dims [0, 512): wave w takes tokens [T w, T w + T) with T = 32 / NW, one instruction per token: 64 lanes x
//     16 bytes = the token's 1024 bytes, written to its padded LDS row. The row address is moved to scalar registers
//     with readlane, so each lane adds only its fixed 16-byte offset.
//   * rope dims [512, 576): whole 128-byte rope rows, 16 bytes a lane (below).
template <int NW, bool KV8>
__device__ __forceinline__ void issue_tile(uint64_t rows, lds_char_ptr tile, int32_t w, int lane) {
    constexpr int kTpw = kTile / NW;
    const uint32_t alo = uint32_t(rows), ahi = uint32_t(rows >> 32);
    if constexpr (KV8) {
        // fp8 latent rows (576 one-byte codes): one instruction per token, all 64 lanes loading 16 bytes each into
        // [kFp8Off, kRowV) of the token's LDS row: lanes 0..35 the codes, lanes 36..63 a second copy of the row's
        // first 448 bytes into the row's tail, which the widening overwrites (and whose last 32 bytes are padding).
        // widen_tile_fp8 turns the codes into the bf16 layout. (Masking lanes 36..63 instead put the loads under a
        // branch, and the compiler's wait-count pass then waited for every tile in flight at that point of the loop.)
#pragma unroll
        for (int i = 0; i < kTpw; ++i) {
            const int32_t t = kTpw * w + i;                                      // wave-uniform
            const uint64_t base = (uint64_t(uint32_t(__builtin_amdgcn_readlane(ahi, t))) << 32) |
                                  uint32_t(__builtin_amdgcn_readlane(alo, t));
            const int32_t piece = lane < kD / 16 ? lane : lane - kD / 16;
            const char* src = reinterpret_cast<const char*>(base) + uint32_t(16 * piece);
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(tile + kRowV * t + kFp8Off), 16, 0,
                                             kLatentCpol);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kTpw; ++i) {
        const int32_t t = kTpw * w + i;                                          // wave-uniform
        const uint64_t base = (uint64_t(uint32_t(__builtin_amdgcn_readlane(ahi, t))) << 32) |
                              uint32_t(__builtin_amdgcn_readlane(alo, t));
        const char* src = reinterpret_cast<const char*>(base) + uint32_t(16 * lane);
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(tile + kRowV * t), 16, 0, kLatentCpol);
    }
    // rope dims: 16-byte loads, 8 lanes per token (a 128-byte rope row), lane l of an instruction filling stored
    // piece l % 8 of token first + l / 8 from the matching logical piece (l % 8) ^ g(t): 8 tokens per instruction, the
    // tile's 4 instructions taken by the first waves (kRopeWaves of them, the same number each).
    constexpr int kRopeWaves = NW < 4 ? NW : 4;
    constexpr int kRInstr = 4 / kRopeWaves;
    if (NW <= 4 || w < kRopeWaves) {                                            // (every wave when NW <= 4)
#pragma unroll
        for (int i = 0; i < kRInstr; ++i) {
            const int32_t first = 8 * (kRInstr * w + i);                         // wave-uniform
            const int32_t t = first + (lane >> 3);
            const uint64_t base = (uint64_t(uint32_t(__shfl(int32_t(ahi), t))) << 32) | uint32_t(__shfl(int32_t(alo), t));
            const char* src = reinterpret_cast<const char*>(base) + 1024 + 16 * ((lane & 7) ^ swz(t));
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(tile + kRegionV + kRowR * first), 16, 0,
                                             kLatentCpol);
        }
    }
}

// Direct-to-LDS loads the waves with the fewest issue per tile: waits leave at most that many of a later tile in flight,
// which for the waves issuing the rope loads as well waits for a little more than needed.
template <int NW, bool KV8>
__device__ __forceinline__ constexpr int tile_loads() {
    return KV8 ? kTile / NW : kTile / NW + (NW <= 4 ? 4 / NW : 0);
}

// fp8 tiles: widen the rows this wave loaded (tokens [32 w / NW, +32 / NW)) from the E4M3 codes at [kFp8Off, +576)
// of each row to the bf16 layout the products read: value dims [0, 512) at the start of the row, rope dims in the
// swizzled rope row. Sixteen lanes a token, each taking 32 value codes and 4 rope codes; every read of a pass is done
// before its writes (they depend on the read data), so the in-place overlap of source and destination is safe. The
// conversion is exact (E4M3 values are bf16 values); the descale is applied in fp32 elsewhere.
template <int NW>
__device__ __forceinline__ void widen_tile_fp8(lds_char_ptr tile, int32_t w, int lane) {
    constexpr int kTpw = kTile / NW;
    const int32_t j = lane & 15;
#pragma unroll
    for (int pass = 0; pass < kTpw / 4; ++pass) {
        const int32_t t = kTpw * w + 4 * pass + (lane >> 4);
        // The lane's offsets inside a tile go through an empty asm statement: the compiler then keeps one copy of
        // them and adds each buffer's address where it is used, instead of holding (buffer + offset) for each of the
        // loop's four buffers across the loop (registers that made the 128-head kernel spill, and the spill reloads
        // inside the loop waited for every tile in flight).
        int32_t row_off = kRowV * t, rope_off = kRegionV + kRowR * t + 16 * ((j >> 1) ^ swz(t)) + 8 * (j & 1);
        asm volatile("" : "+v"(row_off), "+v"(rope_off));
        const lds_char_ptr row = tile + row_off;
        const u32x4_t c0 = *(const __attribute__((address_space(3))) u32x4_t*)(row + kFp8Off + 32 * j);
        const u32x4_t c1 = *(const __attribute__((address_space(3))) u32x4_t*)(row + kFp8Off + 32 * j + 16);
        const uint32_t cr = *(const __attribute__((address_space(3))) uint32_t*)(row + kFp8Off + kDv + 4 * j);
        auto wide = [](uint32_t c) __attribute__((always_inline)) {
            return (u32x2_t){__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false)),
                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true))};
        };
        // Each 16-byte piece is stored as soon as it is converted (the reads above all come first), so that only one
        // piece's registers are live at a time.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x2_t a = wide(q < 2 ? c0[2 * q] : c1[2 * (q - 2)]);
            const u32x2_t b = wide(q < 2 ? c0[2 * q + 1] : c1[2 * (q - 2) + 1]);
            *(__attribute__((address_space(3))) u32x4_t*)(row + 64 * j + 16 * q) = (u32x4_t){a[0], a[1], b[0], b[1]};
        }
        *(__attribute__((address_space(3))) u32x2_t*)(tile + rope_off) = wide(cr);
    }
}

// s_waitcnt vmcnt(n) with the other counters at their maximum (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads and writes have completed (the other counters at their maximum).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wait until at most the loads of kAhead - 1 tiles are outstanding (the counter saturates at 63: with one or two
// waves a little more than the oldest tile is waited for).
// fp8 tiles: also the next tile (it is widened during this step), so at most kAhead - 2 tiles stay outstanding.
template <int NW, bool KV8>
__device__ __forceinline__ void wait_tile() {
    constexpr int kN = (kAhead - (KV8 ? 2 : 1)) * tile_loads<NW, KV8>();
    wait_vmcnt<(kN < 63 ? kN : 63)>();
}

// Scheduling groups of the output product: AHEAD LDS reads, then G groups of M MFMAs, each but the last followed by R
// reads.
template <int M, int G, int AHEAD, int R>
__device__ __forceinline__ void sched_pv() {
    constexpr int kDsRead = 0x100, kMfma = 0x008;
    __builtin_amdgcn_sched_group_barrier(kDsRead, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < G - 1; ++i) {
        __builtin_amdgcn_sched_group_barrier(kMfma, M, 0);
        __builtin_amdgcn_sched_group_barrier(kDsRead, R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, M, 0);
}

// Workgroup barrier without the memory fences of __syncthreads (those would drain the tiles in flight); the empty
// asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace

// Plan: every unit ranked by its token count, longest first (ties in unit order), into p.order.
__global__ __launch_bounds__(256) void mla_plan_kernel(const MlaParams p) {
    __shared__ __attribute__((aligned(16))) int32_t s_len[kMaxPlanUnits];
    __shared__ int32_t s_part[256];
    const int32_t n = p.n_units;
    const int32_t npad = rank_padded(n);
    // Tokens of unit u = ((b S + s) unit_tokens + qtok) n_chunks + c: its chunk's share of the stripe, 0 when the row
    // has no query token qtok (no attention work).
    const int32_t ut = p.unit_tokens, nch = p.n_chunks, ch = p.chunk_tokens;
    for_each_plan_pair(p.q_row_start, p.ctx_len, p.B, p.S, p.T, p.max_row_tokens, p.ctx_cap, p.stripe_begin, p.P,
                       p.geo.interleave, [&](int32_t bs, int32_t ntok, int32_t lr) {
                           for (int32_t qtok = 0; qtok < ut; ++qtok)
                               for (int32_t c = 0; c < nch; ++c)
                                   s_len[(bs * ut + qtok) * nch + c] = qtok < ntok ? max(0, min(lr - c * ch, ch)) : 0;
                       });
    for (int32_t v = n + int32_t(threadIdx.x); v < npad; v += blockDim.x) s_len[v] = -1;
    __syncthreads();
    rank_longest_first(s_len, s_part, n, p.order);
}

// One workgroup per (unit, group of 16 NW heads); wave w of group hg owns heads hg 16 NW + 16 w + [0, 16).
template <int NW, bool REDO, bool KV8>
__global__ __launch_bounds__(64 * NW, 1) void mla_decode_kernel(const MlaParams p) {
    // Four tile buffers as separate arrays: a read of one and a tile load into another then refer to different
    // objects, which the wait-count pass needs to see to leave the other tiles' loads in flight.
    __shared__ __attribute__((aligned(16))) char s_tile0[kTileBytes];
    __shared__ __attribute__((aligned(16))) char s_tile1[kTileBytes];
    __shared__ __attribute__((aligned(16))) char s_tile2[kTileBytes];
    __shared__ __attribute__((aligned(16))) char s_tile3[kTileBytes];
    __shared__ __attribute__((aligned(16))) char s_prob[NW * 1024];   // probabilities of head group w at 1024 w
    __shared__ int32_t s_pages[kMaxChunkPages];
    __shared__ float s_rowsum[16 * NW];
    __shared__ int32_t s_over[NW];
    constexpr int kDB = 32 / NW;                           // 16-dim output blocks of a wave
    const int lane = threadIdx.x & 63;
    const int32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t blk = blockIdx.x;

    if (blk >= p.work_blocks) {                             // padding-token fill role
        if (REDO) return;
        const int32_t k = blk - p.work_blocks;
        const int32_t first = min(max(p.q_row_start[p.B], 0), p.T);
        const int32_t t0 = max(k * p.pad_tokens_per_block, first);
        const int32_t t1 = min((k + 1) * p.pad_tokens_per_block, p.T);
        if (t0 < t1)
            fill_padding(p.out, p.o_ss, p.o_st, p.o_sh, p.lse, p.l_ss, p.l_st, p.S, p.Hq, kDv, t0, t1, threadIdx.x,
                         blockDim.x, p.pad_lse_only);
        return;
    }
    const int32_t rank = blk, hg = 0;                       // one workgroup serves all query heads of a unit
    if (rank >= p.n_units) return;
    // Redo flags are indexed by workgroup: every workgroup of the first launch clears its own here (early-exit units
    // included) and sets it below when its scores outgrew the reference, so a workgroup of the redo launch needs one
    // load to know whether it has anything to do.
    if (!REDO && threadIdx.x == 0) p.ws_redo[rank] = 0;
    if (REDO && !p.ws_redo[rank]) return;
    const int32_t u = p.order ? __builtin_amdgcn_readfirstlane(((const_i32_ptr)p.order)[rank]) : rank;
    const Unit x = decode_unit(p, u);
    if (!REDO && x.c == 0 && x.qtok == p.unit_tokens - 1)
        fill_excess_tokens(p.out + int64_t(x.s) * p.o_ss, p.o_st, p.o_sh, p.lse + int64_t(x.s) * p.l_ss, p.l_st, x.tok0,
                           x.tok1, p.max_row_tokens, p.Hq, kDv, threadIdx.x, blockDim.x, p.pad_lse_only);
    if (!x.live) return;
    const int32_t n16 = lane & 15, c4 = lane >> 4;
    const int32_t hw = hg * 16 * NW + 16 * w;               // first query head of this wave

    if (x.j0 >= x.j1) {
        if (x.c != 0) return;                               // a chunk past the stripe's end: no record is read
        // Empty stripe: (0, -inf) for this wave's heads.
        for (int32_t hh = 0; hh < 16; ++hh) {
            float* o = p.out + int64_t(x.s) * p.o_ss + int64_t(x.t) * p.o_st + int64_t(hw + hh) * p.o_sh;
            for (int32_t d = lane; d < kDv; d += 64) o[d] = 0.f;
        }
        if (lane < 16) p.lse[int64_t(x.s) * p.l_ss + int64_t(x.t) * p.l_st + hw + lane] = neg_inf();
        return;
    }

    const int32_t r = p.stripe_begin + x.s;
    const char* kv_r = p.kv + (int64_t(r) * p.geo.s_stripe << (KV8 ? 0 : 1));
    const int32_t* bt_row = p.bt + int64_t(x.b) * p.bt_stride;
    const int32_t j_last = x.j1 - 1;
    const int32_t ntiles = (x.j1 - x.j0 + kTile - 1) / kTile;

    // Query operand of the score product: head hw + n16, dims [32 ks + 8 c4, +8).
    u32x4_t qreg[kKSteps];
    {
        const uint16_t* qp = p.q + int64_t(x.t) * p.q_st + int64_t(hw + n16) * p.q_sh + 8 * c4;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = *reinterpret_cast<const u32x4_t*>(qp + 32 * ks);
    }

    // The chunk's page ids, staged once in LDS (at most kMaxChunkPages by the choice of chunk length). The barrier's
    // wait also retires the query loads above, so nothing but tile loads is outstanding inside the loop (the
    // wait-count pass would otherwise drain every tile load in flight before the first use of the query operand).
    const int32_t pidx0 = x.j0 >> p.geo.pp_shift;
    {
        const int32_t npages = (j_last >> p.geo.pp_shift) - pidx0 + 1;
        for (int32_t i = threadIdx.x; i < npages; i += 64 * NW) s_pages[i] = bt_row[pidx0 + i];
        __syncthreads();
    }

    // Per-lane LDS byte offsets inside a tile (each read adds a compile-time immediate):
    //   score operand, dims [0, 512): token 16 tb + n16, bytes 64 ks + 16 c4 of its row;
    //   score operand, rope dims: token 16 tb + n16, stored piece (4 k' + c4) ^ g(t) of its rope row (k' = ks - 16);
    //   value operand through transposed reads (ds_read_b64_tr_b16): in each 16-lane group, lane s supplies four
    //   consecutive values of one row and lane q receives element q % 4 of rows q / 4, 4 + q / 4, 8 + q / 4, 12 + q / 4.
    //   Lane s of group c4 points at token 16 r + 4 c4 + s / 4, dims 16 b + 4 (s % 4) (read r = 0, 1 of dim block b),
    //   so lane q receives dim 16 b + q of tokens 8 c4 + e in k order: the B operand, with no permutes. The wave's
    //   dim blocks are b = kDB w + [0, kDB).
    //   Only the token-block-0 offsets live in registers: token block 1 is 16 rows further (a constant), and its rope
    //   swizzle g(t + 16) = g(t) ^ 4 swaps the two pieces k = 0, 1 of block 0.
    const int32_t kofs_v = kRowV * n16 + 16 * c4;
    int32_t kofs_r[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) kofs_r[k] = kRegionV + kRowR * n16 + 16 * ((4 * k + c4) ^ swz(n16));
    const int32_t vofs = kRowV * (4 * c4 + (n16 >> 2)) + 8 * (n16 & 3) + 32 * kDB * w;
    const lds_char_ptr prob_r = (lds_char_ptr)s_prob + 16 * lane;   // + 1024 hg: head group hg's probabilities
    // Buffer b of the ring, b a compile-time constant.
    auto tile_buf = [&](auto bc) __attribute__((always_inline)) -> lds_char_ptr {
        constexpr int b = decltype(bc)::value % kBufs;
        return b == 0 ? (lds_char_ptr)s_tile0 : b == 1 ? (lds_char_ptr)s_tile1 : b == 2 ? (lds_char_ptr)s_tile2
                                                                                   : (lds_char_ptr)s_tile3;
    };

    const int32_t last_tile0 = x.j0 + (ntiles - 1) * kTile;

    // Softmax reference. Each head's probabilities are taken relative to a fixed reference m: the maximum of the
    // unit's first tile. Later tiles may exceed it by up to kRefSlack (log2 units) without any rescaling of the
    // accumulators (p <= 2^64 and sums of such values stay far inside the fp32 and bf16 range), so they are written
    // only by MFMAs and stay in the accumulation registers. Should a head's scores rise further, the workgroup leaves
    // its outputs unwritten, records the exact maxima and a redo flag, and the REDO launch of this kernel computes the
    // unit again with the exact maxima as references.
    constexpr float kRefSlack = 15.0f;
    float m = REDO ? p.ws_max[int64_t(u) * p.Hq + hw + n16] : neg_inf();
    // l: the fp32 sum of the probabilities (for the LSE); lr: the sum of the bf16-rounded probabilities that the value
    // product actually weights by (for the normalisation, so that the applied weights sum to one).
    float m_seen = neg_inf(), l = 0.f, lr = 0.f;
    bool over = false;
    f32x4_t o[32];        // o[kDB hg + b][i]: head 16 hg + 4 c4 + i, dim 16 (kDB w + b) + n16 (unnormalised)
#pragma unroll
    for (int b = 0; b < 32; ++b) o[b] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    {
        // kAhead tiles in flight before the loop; every iteration issues one more (tile indices past the end re-read
        // the last tile into a buffer nobody reads), so the wait at the top of an iteration leaves exactly the
        // kAhead - 1 newest tiles' loads outstanding.
        // The prologue's loads take their LDS address through an opaque copy of the buffer pointer, so the
        // compiler's wait-count pass does not track them against the buffer arrays; tracked, their state merged into
        // the loop header's and made it wait for every load in flight there (a full drain every fourth tile). The
        // explicit wait and barrier at the top of each step order them before the reads of their tiles all the same.
        auto opaque = [](lds_char_ptr t) __attribute__((always_inline)) {
            asm volatile("" : "+v"(t));
            return t;
        };
        const lds_i32_ptr pages = (lds_i32_ptr)s_pages;
        issue_tile<NW, KV8>(token_rows<KV8>(p, pages, pidx0, x.j0, j_last, kv_r, lane),
                            opaque(tile_buf(std::integral_constant<int, 0>{})), w, lane);
        issue_tile<NW, KV8>(token_rows<KV8>(p, pages, pidx0, min(x.j0 + kTile, last_tile0), j_last, kv_r, lane),
                            opaque(tile_buf(std::integral_constant<int, 1>{})), w, lane);
        issue_tile<NW, KV8>(token_rows<KV8>(p, pages, pidx0, min(x.j0 + 2 * kTile, last_tile0), j_last, kv_r, lane),
                            opaque(tile_buf(std::integral_constant<int, 2>{})), w, lane);
        static_assert(kAhead == 3 && kBufs == 4, "ring");
        if constexpr (KV8) {                        // tile 0 is widened before the first step's barrier
            constexpr int kN0 = (kAhead - 1) * tile_loads<NW, KV8>();
            wait_vmcnt<(kN0 < 63 ? kN0 : 63)>();
            asm volatile("" ::: "memory");          // (the LDS reads of the widening stay after the wait)
            widen_tile_fp8<NW>(opaque(tile_buf(std::integral_constant<int, 0>{})), w, lane);
        }

        // Compute tile kt from `tile`.
        auto tile_compute = [&](lds_char_ptr tile, int32_t kt) __attribute__((always_inline)) {
            const int32_t tile0 = x.j0 + kt * kTile;
            const bool tail = tile0 + kTile > x.j1;
            // This tile's lane base addresses, formed once so that every read below carries its remaining offset as
            // an instruction immediate.
            const lds_char_ptr kb_v = tile + kofs_v, kb_r0 = tile + kofs_r[0], kb_r1 = tile + kofs_r[1];
            const lds_char_ptr vb = tile + vofs;

            // Scores S^T[token 16 tb + 4 c4 + i][head n16].
            f32x4_t sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            // Key operand j = 2 ks + tb, read in pairs: the next pair's reads are issued before the current pair's
            // MFMAs and fenced there, so each read overlaps two MFMAs. Left to itself the scheduler waited for every
            // read right before its MFMA; deeper blocks do not fit the registers (128 accumulators and 72 query
            // registers per wave) without spilling. Measured on the 128-head workload: 0.490 -> 0.470 ms.
            auto kop = [&](int j) __attribute__((always_inline)) {
                const int ks = j >> 1, tb = j & 1;
                const lds_char_ptr a = ks < 16 ? kb_v + 16 * kRowV * tb + 64 * ks
                                               : ((ks - 16) ^ tb ? kb_r1 : kb_r0) + 16 * kRowR * tb;
                return *(const __attribute__((address_space(3))) u32x4_t*)a;
            };
            constexpr int KB = 2;
            constexpr int kOps = 2 * kKSteps;
            static_assert(kOps % KB == 0, "whole blocks");
            u32x4_t kcur[KB], knxt[KB];
#pragma unroll
            for (int i = 0; i < KB; ++i) kcur[i] = kop(i);
#pragma unroll
            for (int j0 = 0; j0 < kOps; j0 += KB) {
                if (j0 + KB < kOps) {
#pragma unroll
                    for (int i = 0; i < KB; ++i) knxt[i] = kop(j0 + KB + i);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < KB; ++i) {
                    const int j = j0 + i;
                    sacc[j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[i]), as_bf16x8(qreg[j >> 1]),
                                                                          sacc[j & 1], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < KB; ++i) kcur[i] = knxt[i];
            }

            // Probabilities against the fixed reference.
            float sv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = sacc[e >> 2][e & 3] * p.scale_log2;
                if (tail && tile0 + 16 * (e >> 2) + 4 * c4 + (e & 3) >= x.j1) v = neg_inf();
                sv[e] = v;
            }
            float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                             fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            m_seen = fmaxf(m_seen, mx);
            if (!REDO && kt == 0) m = mx;           // the first tile always holds a real token
            over |= mx > m + kRefSlack;
            u32x4_t pa;
            {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fminf(sv[e] - m, kRefSlack));
#pragma unroll
                for (int d = 0; d < 4; ++d) pa[d] = pack2_f16(pv[2 * d], pv[2 * d + 1]);
                l += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
                const f16x8_t ph = __builtin_bit_cast(f16x8_t, pa);
                float pr[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = float(ph[e]);
                lr += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
            }

            // Share the probabilities: every wave needs all head groups' for its dim slice.
            *(__attribute__((address_space(3))) u32x4_t*)(prob_r + 1024 * w) = pa;
            wait_lgkm0();
            lds_barrier();

            // Values: kDB output blocks of 16 dims for each of the NW head groups; one block's operand from two
            // transposed reads, one head group's from one 16-byte read.
            auto vop = [&](int b) __attribute__((always_inline)) {
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vb + 32 * b));
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vb + 16 * kRowV + 32 * b));
                return bf16x8_to_f16(
                    __builtin_bit_cast(u32x4_t, (s16x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}));
            };
            auto pop = [&](int hg) __attribute__((always_inline)) {
                return __builtin_bit_cast(f16x8_t, *(const __attribute__((address_space(3))) u32x4_t*)(prob_r + 1024 * hg));
            };
            if constexpr (NW >= 8) {                // hold the kDB value operands, stream the head groups
                f16x8_t vv[kDB];
#pragma unroll
                for (int b = 0; b < kDB; ++b) vv[b] = vop(b);
#pragma unroll
                for (int hg = 0; hg < NW; ++hg) {
                    const f16x8_t a = pop(hg);
#pragma unroll
                    for (int b = 0; b < kDB; ++b)
                        o[kDB * hg + b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, vv[b], o[kDB * hg + b], 0, 0, 0);
                }
                sched_pv<kDB, NW, 2 * kDB + 2, 1>();  // value operands and two head groups ahead, then one read per group
            } else {                                // hold the NW probability operands, stream the value blocks
                f16x8_t pp[NW];
#pragma unroll
                for (int hg = 0; hg < NW; ++hg) pp[hg] = pop(hg);
#pragma unroll
                for (int b = 0; b < kDB; ++b) {
                    const f16x8_t v = vop(b);
#pragma unroll
                    for (int hg = 0; hg < NW; ++hg)
                        o[kDB * hg + b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pp[hg], v, o[kDB * hg + b], 0, 0, 0);
                }
                sched_pv<NW, kDB, NW + 4, 2>();       // probabilities and two value blocks ahead, then one block per group
            }
        };

        // One iteration with buffer b (compile time): wait for tile kt, issue the loads of tile kt + kAhead into
        // buffer b + kAhead, compute tile kt from buffer b.
        auto step = [&](auto bc, int32_t kt) __attribute__((always_inline)) {
            constexpr int b = decltype(bc)::value;
            // This wave's pieces of tile kt are in LDS: the loads of the kAhead - 1 newer tiles may stay in flight.
            wait_tile<NW, KV8>();
            wait_lgkm0();                           // this wave's reads of tile kt - 1 and of the probabilities are done
            lds_barrier();                          // ... and every wave's: tile kt - 1's buffer is free
            const int32_t tn0 = min(x.j0 + (kt + kAhead) * kTile, last_tile0);
            issue_tile<NW, KV8>(token_rows<KV8>(p, pages, pidx0, tn0, j_last, kv_r, lane),
                                tile_buf(std::integral_constant<int, b + kAhead>{}), w, lane);
            // fp8: widen this wave's rows of tile kt + 1 (loaded); the next step's barrier publishes them. Fenced from
            // the compute in the instruction schedule: interleaved, both sets of temporaries are live and spill.
            if constexpr (KV8) {
                widen_tile_fp8<NW>(tile_buf(std::integral_constant<int, b + 1>{}), w, lane);
                __builtin_amdgcn_sched_barrier(0);
            }
            tile_compute(tile_buf(std::integral_constant<int, b>{}), kt);
        };
        for (int32_t kt = 0; kt < ntiles; kt += kBufs) {
            step(std::integral_constant<int, 0>{}, kt);
            if (kt + 1 >= ntiles) break;
            step(std::integral_constant<int, 1>{}, kt + 1);
            if (kt + 2 >= ntiles) break;
            step(std::integral_constant<int, 2>{}, kt + 2);
            if (kt + 3 >= ntiles) break;
            step(std::integral_constant<int, 3>{}, kt + 3);
        }
        wait_vmcnt<0>();                            // the over-issued tail loads land before the waves retire
    }
    if (!REDO) {
        // A workgroup-wide decision, so that every wave takes the same path.
        // The vote is taken by the whole wave, before the one-lane store: inside `lane == 0` it would see lane 0 only.
        const bool wave_over = __any(over);
        if (lane == 0) s_over[w] = wave_over ? 1 : 0;
        __syncthreads();
        int32_t any_over = 0;
#pragma unroll
        for (int v = 0; v < NW; ++v) any_over |= s_over[v];
        if (threadIdx.x == 0) p.ws_redo[rank] = any_over;
        if (any_over) {
            if (c4 == 0) p.ws_max[int64_t(u) * p.Hq + hw + n16] = m_seen;
            return;
        }
    }

    // Epilogue: row sums over the four lane groups (each head's sum lives in the wave that scored it, and goes to LDS
    // for the waves holding that head's dims), then the normalised partial or this chunk's record.
    const bool split = p.n_chunks > 1 && x.Lr > p.chunk_tokens;
    float* rec = split ? p.ws_rec + int64_t(u) * p.rec_floats : nullptr;
    float ls = l, lrs = lr;
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    lrs += __shfl_xor(lrs, 16);
    lrs += __shfl_xor(lrs, 32);
    if (c4 == 0) s_rowsum[hw + n16] = lrs;
    __syncthreads();
    // Lane base: head 4 c4 (+ 16 hg + i), dim 16 kDB w + n16 (+ 16 b); head stride of the partial or of the record.
    const int64_t hs = split ? int64_t(kDv) : p.o_sh;
    float* const base = (split ? rec : p.out + int64_t(x.s) * p.o_ss + int64_t(x.t) * p.o_st) + 4 * c4 * hs +
                        16 * kDB * w + n16;
#pragma unroll
    for (int hg = 0; hg < NW; ++hg) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float li = s_rowsum[16 * hg + 4 * c4 + i];
            const float inv = (split ? 1.0f : (li > 0.f ? 1.0f / li : 0.f)) * p.v_scale;
            float* dst = base + (16 * hg + i) * hs;
#pragma unroll
            for (int b = 0; b < kDB; ++b) dst[16 * b] = o[kDB * hg + b][i] * inv;
        }
    }
    if (c4 == 0) {
        const int32_t h = hw + n16;
        if (split) {
            rec[int64_t(p.Hq) * kDv + h] = m;
            rec[int64_t(p.Hq) * kDv + p.Hq + h] = ls;
            rec[int64_t(p.Hq) * kDv + 2 * p.Hq + h] = lrs;
        } else {
            p.lse[int64_t(x.s) * p.l_ss + int64_t(x.t) * p.l_st + h] = ls > 0.f ? (m + log2f(ls)) * kLn2 : neg_inf();
        }
    }
}

// Exact merge of the chunk records of every (row, stripe, query token) whose stripe spans several chunks:
// with M = max_c m_c, o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) lr_c and lse = (M + log2 sum_c 2^(m_c - M) l_c) ln 2
// (l_c the fp32 sum of a chunk's probabilities, lr_c the sum of their bf16 roundings that o_c was weighted by).
// One block of 256 threads per (item, pair of heads); thread i handles head 2 blk + i / 128, dims [4 (i % 128), +4).
__global__ __launch_bounds__(256) void mla_chunk_merge_kernel(const MlaParams p) {
    const int32_t hpairs = p.Hq / 2;
    const int32_t item = blockIdx.x / hpairs;
    const int32_t h = 2 * (blockIdx.x % hpairs) + (threadIdx.x >> 7);
    const int32_t d4 = threadIdx.x & 127;
    const Unit x = decode_unit(p, item * p.n_chunks);
    if (!x.live || x.Lr <= p.chunk_tokens) return;      // written directly
    const int32_t nch = (x.Lr + p.chunk_tokens - 1) / p.chunk_tokens;
    const float* rec0 = p.ws_rec + int64_t(item) * p.n_chunks * p.rec_floats;
    float M = neg_inf();
    for (int32_t c = 0; c < nch; ++c) M = fmaxf(M, rec0[c * p.rec_floats + int64_t(p.Hq) * kDv + h]);
    float Lsum = 0.f, Lr = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int32_t c = 0; c < nch; ++c) {
        const float* rc = rec0 + c * p.rec_floats;
        const float wgt = exp2f(rc[int64_t(p.Hq) * kDv + h] - M);
        Lsum += wgt * rc[int64_t(p.Hq) * kDv + p.Hq + h];
        Lr += wgt * rc[int64_t(p.Hq) * kDv + 2 * p.Hq + h];
        acc += wgt * *reinterpret_cast<const f32x4_t*>(rc + int64_t(h) * kDv + 4 * d4);
    }
    const float inv = Lr > 0.f ? 1.0f / Lr : 0.f;
    float* o = p.out + int64_t(x.s) * p.o_ss + int64_t(x.t) * p.o_st + int64_t(h) * p.o_sh + 4 * d4;
    *reinterpret_cast<f32x4_t*>(o) = acc * inv;
    if (d4 == 0) p.lse[int64_t(x.s) * p.l_ss + int64_t(x.t) * p.l_st + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : neg_inf();
}

// ------------------------------------------------------------------------------------------------------------ host
namespace {

struct MlaShape {
    int64_t n_items, n_chunks, chunk_tokens, n_units, rec_floats;
    int64_t nw, head_groups, work_blocks;
    bool plan;
};

MlaShape mla_shape(const cp_paged_args& a) {
    MlaShape d{};
    const int64_t mrt = std::max<int64_t>(1, a.max_row_tokens);
    d.n_items = int64_t(a.num_rows) * a.stripe_count * mrt;
    const int64_t max_lr = max_stripe_length(a);
    int64_t nch = 1;
    if (d.n_items > 0 && d.n_items < kTargetUnits && max_lr > 256) {
        nch = std::min<int64_t>((kTargetUnits + d.n_items - 1) / d.n_items, (max_lr + 255) / 256);
        nch = std::max<int64_t>(nch, 1);
    }
    int64_t ch = std::max<int64_t>(kTile, (max_lr + nch - 1) / nch);
    ch = (ch + kTile - 1) / kTile * kTile;
    // A chunk's page ids must fit the LDS staging area: at most kMaxChunkPages pages of page_size / P slots.
    const int64_t pp = std::max<int64_t>(1, a.page_size / std::max(1, a.num_partners));
    ch = std::min<int64_t>(ch, (kMaxChunkPages - 1) * pp / kTile * kTile);
    d.chunk_tokens = ch;
    d.n_chunks = std::max<int64_t>(1, (max_lr + ch - 1) / ch);
    d.n_units = d.n_items * d.n_chunks;
    d.rec_floats = int64_t(a.num_q_heads) * (kDv + 3);
    d.plan = d.n_units <= kMaxPlanUnits;
    d.nw = std::min<int64_t>(8, a.num_q_heads / 16);
    d.head_groups = 1;
    d.work_blocks = d.n_units;
    return d;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool mla_decode_eligible(const cp_paged_args& a, const PoolGeom& geo) {
    if (a.kind != CPATTN_MLA || a.dtype != CPATTN_BF16 || a.head_dim != kD || a.head_dim_v != kDv) return false;
    const bool kv8 = a.kv_format == CPATTN_KV_FP8_E4M3;
    if (a.num_q_heads != 16 && a.num_q_heads != 32 && a.num_q_heads != 64 && a.num_q_heads != 128) return false;
    if (geo.pp_shift < 0) return false;
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    if (!al16(a.q) || !al16(a.k_pool) || !al16(a.out)) return false;
    if ((a.q_stride_token | a.q_stride_head) & 7) return false;
    if ((a.kv_stride_stripe | a.kv_stride_page | a.kv_stride_slot) & (kv8 ? 15 : 7)) return false;   // 16-byte rows
    if ((a.out_stride_stripe | a.out_stride_token | a.out_stride_head) & 3) return false;
    const MlaShape d = mla_shape(a);
    if (d.work_blocks + (a.num_tokens + 3) / 4 > (int64_t(1) << 31) - 1) return false;
    return true;
}

// Workspace: [unit order (plan)] [chunk records (split stripes)] [redo flags] [score maxima of units to redo].
struct MlaWorkspace {
    int64_t order, rec, redo, max, total;
};

MlaWorkspace mla_workspace(const MlaShape& d, int64_t hq) {
    MlaWorkspace w{};
    w.order = 0;
    w.rec = d.plan ? align256(4 * d.n_units) : 0;
    w.redo = w.rec + (d.n_chunks > 1 ? align256(d.n_units * d.rec_floats * 4) : 0);
    w.max = w.redo + align256(4 * d.n_units * d.head_groups);
    w.total = w.max + align256(4 * d.n_units * hq);
    return w;
}

int64_t mla_decode_workspace_bytes(const cp_paged_args& a) {
    const MlaShape d = mla_shape(a);
    return d.n_units > 0 ? mla_workspace(d, a.num_q_heads).total : 0;
}

// The kernel instance for NW waves, the redo role and the pool element type.
template <bool REDO>
void launch_mla_variant(int64_t nw, bool kv8, dim3 grid, hipStream_t stream, const MlaParams& p) {
    auto go = [&](auto nwc, auto k8) {
        constexpr int NW = decltype(nwc)::value;
        constexpr bool K8 = decltype(k8)::value;
        hipLaunchKernelGGL((mla_decode_kernel<NW, REDO, K8>), grid, dim3(64 * NW), 0, stream, p);
    };
    using T8 = std::true_type;
    using F8 = std::false_type;
    switch (nw) {
        case 1: kv8 ? go(std::integral_constant<int, 1>{}, T8{}) : go(std::integral_constant<int, 1>{}, F8{}); break;
        case 2: kv8 ? go(std::integral_constant<int, 2>{}, T8{}) : go(std::integral_constant<int, 2>{}, F8{}); break;
        case 4: kv8 ? go(std::integral_constant<int, 4>{}, T8{}) : go(std::integral_constant<int, 4>{}, F8{}); break;
        default: kv8 ? go(std::integral_constant<int, 8>{}, T8{}) : go(std::integral_constant<int, 8>{}, F8{}); break;
    }
}

int32_t launch_mla_decode(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream) {
    const MlaShape d = mla_shape(a);
    MlaParams p{};
    p.q = static_cast<const uint16_t*>(a.q);
    p.q_st = a.q_stride_token;
    p.q_sh = a.q_stride_head;
    p.kv = static_cast<const char*>(a.k_pool);
    p.geo = geo;
    p.q_row_start = a.q_row_start;
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
    char* ws = static_cast<char*>(a.workspace);
    const MlaWorkspace wl = mla_workspace(d, a.num_q_heads);
    p.order = d.plan && d.n_units > 0 ? reinterpret_cast<int32_t*>(ws + wl.order) : nullptr;
    p.ws_rec = d.n_chunks > 1 ? reinterpret_cast<float*>(ws + wl.rec) : nullptr;
    p.ws_redo = d.n_units > 0 ? reinterpret_cast<int32_t*>(ws + wl.redo) : nullptr;
    p.ws_max = d.n_units > 0 ? reinterpret_cast<float*>(ws + wl.max) : nullptr;
    p.rec_floats = d.rec_floats;
    p.B = a.num_rows;
    p.T = a.num_tokens;
    p.P = a.num_partners;
    p.stripe_begin = a.stripe_begin;
    p.S = a.stripe_count;
    p.Hq = a.num_q_heads;
    p.max_pages = a.max_pages;
    p.ctx_cap = ctx_cap_of(a);
    p.page_size = a.page_size;
    p.max_row_tokens = a.max_row_tokens;
    p.unit_tokens = std::max(1, a.max_row_tokens);
    p.n_chunks = int32_t(d.n_chunks);
    p.chunk_tokens = int32_t(d.chunk_tokens);
    p.n_units = int32_t(d.n_units);
    p.pad_tokens_per_block = 4;
    p.pad_blocks = (a.num_tokens + 3) / 4;
    p.head_groups = int32_t(d.head_groups);
    p.work_blocks = int32_t(d.work_blocks);
    const bool kv8 = a.kv_format == CPATTN_KV_FP8_E4M3;
    p.scale_log2 = a.scale * (kv8 ? a.k_descale : 1.0f) * kLog2e;
    p.v_scale = kv8 ? a.v_descale : 1.0f;
    p.pad_lse_only = (a.flags & CPATTN_FLAG_PAD_LSE_ONLY) ? 1 : 0;

    if (p.order) {
        hipLaunchKernelGGL(mla_plan_kernel, dim3(uint32_t((d.n_units + kRankItems - 1) / kRankItems)), dim3(256), 0, stream,
                           p);
        if (int32_t st = check_launch("cp_paged_attn_partial (MLA plan)")) return st;
    }
    const int64_t blocks = d.work_blocks + p.pad_blocks;
    if (blocks > 0) {
        const dim3 grid{uint32_t(blocks), 1, 1};
        launch_mla_variant<false>(d.nw, kv8, grid, stream, p);
        if (int32_t st = check_launch("cp_paged_attn_partial (MLA decode)")) return st;
    }
    if (d.work_blocks > 0) {                         // workgroups whose scores outgrew their reference, if any
        const dim3 grid{uint32_t(d.work_blocks), 1, 1};
        launch_mla_variant<true>(d.nw, kv8, grid, stream, p);
        if (int32_t st = check_launch("cp_paged_attn_partial (MLA redo)")) return st;
    }
    if (d.n_chunks > 1 && d.n_items > 0) {
        hipLaunchKernelGGL(mla_chunk_merge_kernel, dim3(uint32_t(d.n_items * (a.num_q_heads / 2))), dim3(256), 0,
                           stream, p);
        return check_launch("cp_paged_attn_partial (MLA chunk merge)");
    }
    return CPATTN_OK;
}

}  // namespace cpattn
