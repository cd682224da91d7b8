// bf16 MLA per-stripe paged partial (one latent head: key = the 576-value latent row, value = its first 512 values),
// built for gfx950 MFMA.
//
// What it computes is the partial of one partner over the slots it holds, returned as (out, natural-log lse), with the
// one latent head of MLA shared by all query heads (mstar PR #1124, "Context / Sequence Parallel 1/5", PR description:
// the context-parallel decode covers MLA's single latent head as well as GQA).
//
// Work decomposition. A unit is (row b, stripe s, query token, chunk of the stripe's local tokens). It runs on one
// workgroup of NW <= 4 waves per group of 16 NW query heads (two workgroups for 128 heads); each wave owns 16 heads.
// The latent rows of the unit stream through LDS in tiles of 32 tokens (three buffers, two tiles in flight), loaded
// straight from global memory into LDS, and every wave reads each tile twice: as the key operand of the score product
// and as the value operand of the output product. 16 heads per wave keeps the query operand (72 VGPRs) and the output
// accumulators (128) in registers at one wave per SIMD; 32 heads per wave would halve the LDS reads but does not fit.
// A small plan kernel orders the units longest first, so the hardware's in-order dispatch packs long and short units
// onto the same compute unit. A stripe longer than one chunk leaves one unnormalised record per chunk and a merge
// kernel combines them exactly.
//
// Per tile and wave (16 heads x 32 tokens):
//   * scores S^T[token][head] = K . Q^T with v_mfma_f32_16x16x32_bf16: A = latent rows (token per lane, 8 dims per
//     lane group), B = the wave's query heads, held in registers for the whole unit. 36 MFMAs.
//   * online softmax in log2 units with a lazily moved running max (moved only when a tile maximum exceeds it by more
//     than 8). The running sum adds the fp32 probabilities, so the lse keeps fp32 accuracy; the value product takes
//     them rounded to bf16 (a relative change of at most 2^-9 per weight, which averages out over a stripe's tokens).
//   * out += P . V with v_mfma_f32_16x16x32_bf16: the score layout left by the first product is already the A-operand
//     layout (k index 8c + e of lane group c is tile token 16 (e / 4) + 4c + e % 4), and the B operand of each 16-dim
//     output tile comes from two transposed LDS reads (ds_read_b64_tr_b16), so no register staging or permutes are
//     needed. 32 MFMAs into 128 accumulator registers.
//
// LDS layout of a tile: token t's 72 16-byte pieces at [72t, 72t + 72), piece p stored at 72t + (p ^ g(t)) with
// g(t) = (t ^ (t >> 2)) & 7. Measured on gfx950, both read patterns (sixteen tokens at one piece for the score operand,
// the transposed reads of four tokens for the value operand) then run at the full rate of their instruction; without
// the swizzle the score reads run at a quarter and the value reads at half of it.
#include "launch.h"

namespace cpattn {

namespace {

constexpr int kD = 576;                        // latent row (key) length
constexpr int kDv = 512;                       // value length
constexpr int kTile = 32;                      // tokens per LDS tile
constexpr int kPieces = kD / 8;                // 16-byte pieces per latent row
constexpr int kTileChunks = kTile * kPieces;   // 16-byte pieces per tile
constexpr int kBufs = 3;
constexpr int kKSteps = kD / 32;               // k-steps of the score product
constexpr int kMaxPlanUnits = 1024;            // units sorted by the plan kernel (block order above)
constexpr int kTargetUnits = 512;              // about two units per compute unit before chunks are split

typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;

struct MlaParams {
    const uint16_t* q;
    int64_t q_st, q_sh;
    const uint16_t* kv;
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
    int64_t rec_floats;
    int32_t B, T, P, stripe_begin, S, Hq, max_pages, page_size, max_row_tokens;
    int32_t n_chunks, chunk_tokens, n_units, pad_blocks, pad_tokens_per_block;
    int32_t head_groups, work_blocks;   // workgroups per unit (1 or 2) and blocks before the padding role
    float scale_log2;
};

__device__ __forceinline__ int swz(int t) { return (t ^ (t >> 2)) & 7; }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

struct Unit {
    int32_t b, s, qtok, c;
    int32_t t;           // query token (bucket index)
    int32_t Lr;          // stripe length
    int32_t j0, j1;      // chunk range of local tokens
    bool live;           // the row has this query token
};

__device__ __forceinline__ Unit decode_unit(const MlaParams& p, int32_t u) {
    const const_i32_ptr qrs = (const_i32_ptr)p.q_row_start;
    const const_i32_ptr cl = (const_i32_ptr)p.ctx_len;
    Unit x;
    x.c = u % p.n_chunks;
    int32_t v = u / p.n_chunks;
    x.qtok = v % p.max_row_tokens;
    v /= p.max_row_tokens;
    x.s = v % p.S;
    x.b = v / p.S;
    const int32_t tok0 = min(max(qrs[x.b], 0), p.T);
    const int32_t tok1 = min(max(qrs[x.b + 1], tok0), p.T);
    const int32_t ntok = min(tok1 - tok0, p.max_row_tokens);
    x.live = x.qtok < ntok;
    x.t = tok0 + x.qtok;
    const int32_t L = min(max(cl[x.b], 0), p.max_pages * p.page_size);
    x.Lr = stripe_length(L, p.stripe_begin + x.s, p.P);
    x.j0 = x.c * p.chunk_tokens;
    x.j1 = min(x.j0 + p.chunk_tokens, x.Lr);
    return x;
}

// Tokens of unit u (0 when it does no attention work): the sort key of the plan kernel.
__device__ __forceinline__ int32_t unit_tokens(const MlaParams& p, int32_t u) {
    const int32_t c = u % p.n_chunks;
    int32_t v = u / p.n_chunks;
    const int32_t qtok = v % p.max_row_tokens;
    v /= p.max_row_tokens;
    const int32_t s = v % p.S;
    const int32_t b = v / p.S;
    const int32_t tok0 = min(max(p.q_row_start[b], 0), p.T);
    const int32_t tok1 = min(max(p.q_row_start[b + 1], tok0), p.T);
    if (qtok >= min(tok1 - tok0, p.max_row_tokens)) return 0;
    const int32_t L = min(max(p.ctx_len[b], 0), p.max_pages * p.page_size);
    const int32_t Lr = stripe_length(L, p.stripe_begin + s, p.P);
    return max(0, min(Lr - c * p.chunk_tokens, p.chunk_tokens));
}

// Page ids of a tile, one per lane: lane L holds the block-table entry of tile token L % 32 (tokens past the chunk end
// take its last token). Loaded an iteration before the tile's own loads are issued; checked where used.
__device__ __forceinline__ int32_t load_tile_pages(const MlaParams& p, const int32_t* __restrict__ bt_row,
                                                   int32_t tile0, int32_t j_last, int lane) {
    const int32_t j = min(tile0 + (lane & 31), j_last);
    return bt_row[j >> p.geo.pp_shift];
}

// Issue the direct-to-LDS loads of one tile: wave w's instruction k fills pieces [64 (NW k + w), +64) of the buffer.
// The 64 pieces of one instruction belong to at most two tokens; their page ids come from the tile's page vector with
// readlane, so the page bases are formed on the scalar unit. Tokens past the chunk end re-read its last token (their
// values are masked out).
template <int NW>
__device__ __forceinline__ void issue_tile(const MlaParams& p, int32_t pages, int64_t base_r, int32_t tile0,
                                           int32_t j_last, u32x4_t* buf, int32_t w, int lane) {
    constexpr int kInstr = kTileChunks / (64 * NW);
#pragma unroll
    for (int k = 0; k < kInstr; ++k) {
        const int32_t c0 = 64 * (NW * k + w);                  // wave-uniform
        const int32_t ta = c0 / kPieces;
        const int32_t tb = (c0 + 63) / kPieces;
        int32_t pa = __builtin_amdgcn_readlane(pages, ta);
        int32_t pb = __builtin_amdgcn_readlane(pages, tb);
        pa = (pa >= 0 && pa < p.geo.num_pages) ? pa : 0;
        pb = (pb >= 0 && pb < p.geo.num_pages) ? pb : 0;
        const uint16_t* base_a = p.kv + base_r + int64_t(pa) * p.geo.s_page;
        const uint16_t* base_b = p.kv + base_r + int64_t(pb) * p.geo.s_page;
        const int32_t c = c0 + lane;
        const int32_t t = c / kPieces;
        const int32_t piece = (c - t * kPieces) ^ swz(t);
        const int32_t j = min(tile0 + t, j_last);
        const uint16_t* src = (t == ta ? base_a : base_b) + int64_t(j & (p.geo.pp - 1)) * p.geo.s_slot + 8 * piece;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(buf + c0), 16, 0, 0);
    }
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

}  // namespace

// Plan: rank every unit by its token count, longest first (ties in unit order), into p.order.
__global__ __launch_bounds__(1024) void mla_plan_kernel(const MlaParams p) {
    __shared__ int32_t s_len[kMaxPlanUnits];
    const int32_t n = p.n_units;
    for (int32_t u = threadIdx.x; u < n; u += blockDim.x) s_len[u] = unit_tokens(p, u);
    __syncthreads();
    for (int32_t u = threadIdx.x; u < n; u += blockDim.x) {
        const int32_t mine = s_len[u];
        int32_t rank = 0;
        for (int32_t v = 0; v < n; ++v) {
            const int32_t o = s_len[v];
            rank += (o > mine) || (o == mine && v < u);
        }
        p.order[rank] = u;
    }
}

// One workgroup per (unit, group of 16 NW heads); wave w of group hg owns heads hg 16 NW + 16 w + [0, 16).
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void mla_decode_kernel(const MlaParams p) {
    __shared__ u32x4_t s_buf[kBufs][kTileChunks];
    const int lane = threadIdx.x & 63;
    const int32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t blk = blockIdx.x;

    if (blk >= p.work_blocks) {                             // padding-token fill role
        const int32_t k = blk - p.work_blocks;
        const int32_t first = min(max(p.q_row_start[p.B], 0), p.T);
        const int32_t t0 = max(k * p.pad_tokens_per_block, first);
        const int32_t t1 = min((k + 1) * p.pad_tokens_per_block, p.T);
        if (t0 < t1)
            fill_padding(p.out, p.o_ss, p.o_st, p.o_sh, p.lse, p.l_ss, p.l_st, p.S, p.Hq, kDv, t0, t1, threadIdx.x,
                         blockDim.x);
        return;
    }
    // Block -> (unit rank, head group). With two head groups, the groups of one unit are 8 blocks apart: the same XCD
    // (blocks go round-robin over the 8 XCDs), so the second group's tile reads hit that XCD's L2.
    int32_t rank = blk, hg = 0;
    if (p.head_groups == 2) {
        rank = (blk >> 4) * 8 + (blk & 7);
        hg = (blk >> 3) & 1;
    }
    if (rank >= p.n_units) return;
    const int32_t u = p.order ? __builtin_amdgcn_readfirstlane(((const_i32_ptr)p.order)[rank]) : rank;
    const Unit x = decode_unit(p, u);
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
    const int64_t base_r = int64_t(r) * p.geo.s_stripe;
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

    // Two tiles in flight before the loop; every iteration issues the page ids of tile kt + 3, then the loads of tile
    // kt + 2 (tile indices past the end re-read the last tile into a buffer nobody reads). The wait at the top of an
    // iteration leaves exactly the newest tile's loads outstanding: tile kt and the page ids of tile kt + 2 are in.
    constexpr int kInstr = kTileChunks / (64 * NW);
    const int32_t last_tile0 = x.j0 + (ntiles - 1) * kTile;
    int32_t pages_next;
    {
        const int32_t pg0 = load_tile_pages(p, bt_row, x.j0, j_last, lane);
        const int32_t pg1 = load_tile_pages(p, bt_row, min(x.j0 + kTile, last_tile0), j_last, lane);
        pages_next = load_tile_pages(p, bt_row, min(x.j0 + 2 * kTile, last_tile0), j_last, lane);
        issue_tile<NW>(p, pg0, base_r, x.j0, j_last, s_buf[0], w, lane);
        issue_tile<NW>(p, pg1, base_r, min(x.j0 + kTile, last_tile0), j_last, s_buf[1], w, lane);
    }

    f32x4_t o[32];                                   // o[b][i]: head hw + 4 c4 + i, dim 16 b + n16 (unnormalised)
#pragma unroll
    for (int b = 0; b < 32; ++b) o[b] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    float m = neg_inf(), l = 0.f;

    // Per-lane LDS piece offsets. Score operand: token 16 tb + n16, piece 4 ks + c4 -> 4 ks ^ (c4 ^ g(t)).
    int32_t kofs_even[2], kofs_odd[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int32_t t = 16 * tb + n16;
        const int32_t xg = c4 ^ swz(t);
        kofs_even[tb] = kPieces * t + xg;          // ks even: 4 ks + xg
        kofs_odd[tb] = kPieces * t + (xg ^ 4) - 4; // ks odd: 4 ks - 4 + (xg ^ 4)
    }
    // Value operand through transposed LDS reads (ds_read_b64_tr_b16): in each 16-lane group, lane s supplies four
    // consecutive values of one row and lane q receives element q % 4 of rows q / 4, 4 + q / 4, 8 + q / 4, 12 + q / 4.
    // Lane s of group c4 points at token 16 r + 4 c4 + s / 4, dims 16 b + 4 (s % 4) (read r = 0, 1 of dim block b),
    // so lane q of the group receives dim 16 b + q of tokens 8 c4 + e in k order: the B operand, with no permutes.
    // Byte offset: token t's piece (2 b + (s / 2) % 2) ^ g(t), plus 8 (s % 2); the dim block enters as 2 b ^ y with
    // y = (s / 2) % 2 ^ g(t), which splits into a lane part for b % 4 and an immediate 128 (b / 4).
    int32_t vbase[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int32_t t = 16 * r + 4 * c4 + (n16 >> 2);
        const int32_t y = ((n16 >> 1) & 1) ^ swz(t);
#pragma unroll
        for (int k = 0; k < 4; ++k) vbase[r][k] = 16 * (kPieces * t + ((2 * k) ^ y)) + 8 * (n16 & 1);
    }
    const lds_s16x4_ptr lds_bytes0 = (lds_s16x4_ptr)(s_buf[0]);

    for (int32_t kt = 0; kt < ntiles; ++kt) {
        wait_vmcnt<kInstr>();                       // this wave's pieces of tile kt are in LDS
        lds_barrier();                              // ... and every wave's; tile kt - 1's buffer is free
        {
            const int32_t pages = pages_next;
            pages_next = load_tile_pages(p, bt_row, min(x.j0 + (kt + 3) * kTile, last_tile0), j_last, lane);
            issue_tile<NW>(p, pages, base_r, min(x.j0 + (kt + 2) * kTile, last_tile0), j_last,
                           s_buf[(kt + 2) % kBufs], w, lane);
        }
        const u32x4_t* buf = s_buf[kt % kBufs];
        const int32_t tile0 = x.j0 + kt * kTile;
        const bool tail = tile0 + kTile > x.j1;

        // Scores S^T[token 16 tb + 4 c4 + i][head n16].
        f32x4_t sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int32_t pos = (ks & 1) ? kofs_odd[tb] + 4 * ks : kofs_even[tb] + 4 * ks;
                sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf[pos]), as_bf16x8(qreg[ks]), sacc[tb],
                                                                   0, 0, 0);
            }
        }

        // Online softmax.
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = sacc[e >> 2][e & 3] * p.scale_log2;
            if (tail && tile0 + 16 * (e >> 2) + 4 * c4 + (e & 3) >= x.j1) v = neg_inf();
            sv[e] = v;
        }
        float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__any(mx > m + 8.0f)) {
            const float m_new = fmaxf(m, mx);
            const float alpha = exp2f(m - m_new);     // 0 on the first tile (m = -inf)
            l *= alpha;
            m = m_new;
            float a_o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a_o[i] = __shfl(alpha, 4 * c4 + i);
#pragma unroll
            for (int b = 0; b < 32; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[b][i] *= a_o[i];
        }
        u32x4_t pa;
        {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(sv[e] - m);
#pragma unroll
            for (int d = 0; d < 4; ++d) pa[d] = pack2_bf16(pv[2 * d], pv[2 * d + 1]);
            l += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        }

        // Values: 32 output tiles of 16 dims, each from two transposed reads.
        {
            const int32_t buf_bytes = (kt % kBufs) * kTileChunks * 16;
#pragma unroll
            for (int b = 0; b < 32; ++b) {
                const int32_t imm = buf_bytes + 128 * (b >> 2);
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_ptr)((__attribute__((address_space(3))) char*)lds_bytes0 + vbase[0][b & 3] + imm));
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_ptr)((__attribute__((address_space(3))) char*)lds_bytes0 + vbase[1][b & 3] + imm));
                const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, (s16x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa), bop, o[b], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();                                // the over-issued tail loads land before the waves retire

    // Epilogue: row sums over the four lane groups, then the normalised partial or this chunk's record.
    const bool split = p.n_chunks > 1 && x.Lr > p.chunk_tokens;
    float* rec = split ? p.ws_rec + int64_t(u) * p.rec_floats : nullptr;
    float ls = l;
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t h = hw + 4 * c4 + i;
        const float li = __shfl(ls, 4 * c4 + i);
        const float inv = split ? 1.0f : (li > 0.f ? 1.0f / li : 0.f);
        float* dst = split ? rec + int64_t(h) * kDv
                           : p.out + int64_t(x.s) * p.o_ss + int64_t(x.t) * p.o_st + int64_t(h) * p.o_sh;
#pragma unroll
        for (int b = 0; b < 32; ++b) dst[16 * b + n16] = o[b][i] * inv;
    }
    if (c4 == 0) {
        const int32_t h = hw + n16;
        if (split) {
            rec[int64_t(p.Hq) * kDv + h] = m;
            rec[int64_t(p.Hq) * kDv + p.Hq + h] = ls;
        } else {
            p.lse[int64_t(x.s) * p.l_ss + int64_t(x.t) * p.l_st + h] = ls > 0.f ? (m + log2f(ls)) * kLn2 : neg_inf();
        }
    }
}

// Exact merge of the chunk records of every (row, stripe, query token) whose stripe spans several chunks:
// with M = max_c m_c, o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c and lse = (M + log2 sum_c 2^(m_c - M) l_c) ln 2.
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
    float Lsum = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int32_t c = 0; c < nch; ++c) {
        const float* rc = rec0 + c * p.rec_floats;
        const float wgt = exp2f(rc[int64_t(p.Hq) * kDv + h] - M);
        Lsum += wgt * rc[int64_t(p.Hq) * kDv + p.Hq + h];
        acc += wgt * *reinterpret_cast<const f32x4_t*>(rc + int64_t(h) * kDv + 4 * d4);
    }
    const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
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
    const int64_t max_lr = (int64_t(std::max(a.max_ctx_len, 0)) + a.num_partners - 1) / a.num_partners;
    int64_t nch = 1;
    if (d.n_items > 0 && d.n_items < kTargetUnits && max_lr > 256) {
        nch = std::min<int64_t>((kTargetUnits + d.n_items - 1) / d.n_items, (max_lr + 255) / 256);
        nch = std::max<int64_t>(nch, 1);
    }
    int64_t ch = std::max<int64_t>(kTile, (max_lr + nch - 1) / nch);
    ch = (ch + kTile - 1) / kTile * kTile;
    d.chunk_tokens = ch;
    d.n_chunks = std::max<int64_t>(1, (max_lr + ch - 1) / ch);
    d.n_units = d.n_items * d.n_chunks;
    d.rec_floats = int64_t(a.num_q_heads) * (kDv + 2);
    d.plan = d.n_units <= kMaxPlanUnits;
    d.nw = std::min<int64_t>(4, a.num_q_heads / 16);
    d.head_groups = d.nw > 0 ? a.num_q_heads / (16 * d.nw) : 1;
    d.work_blocks = d.head_groups == 2 ? (d.n_units + 7) / 8 * 16 : d.n_units;
    return d;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool mla_decode_eligible(const cp_paged_args& a, const PoolGeom& geo) {
    if (a.kind != CPATTN_MLA || a.dtype != CPATTN_BF16 || a.head_dim != kD || a.head_dim_v != kDv) return false;
    if (a.num_q_heads != 16 && a.num_q_heads != 32 && a.num_q_heads != 64 && a.num_q_heads != 128) return false;
    if (geo.pp_shift < 0) return false;
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    if (!al16(a.q) || !al16(a.k_pool) || !al16(a.out)) return false;
    if ((a.q_stride_token | a.q_stride_head | a.kv_stride_stripe | a.kv_stride_page | a.kv_stride_slot) & 7) return false;
    if ((a.out_stride_stripe | a.out_stride_token | a.out_stride_head) & 3) return false;
    const MlaShape d = mla_shape(a);
    if (d.work_blocks + (a.num_tokens + 3) / 4 > (int64_t(1) << 31) - 1) return false;
    return true;
}

int64_t mla_decode_workspace_bytes(const cp_paged_args& a) {
    const MlaShape d = mla_shape(a);
    int64_t bytes = d.plan ? align256(4 * d.n_units) : 0;
    if (d.n_chunks > 1) bytes += d.n_units * d.rec_floats * 4;
    return bytes;
}

int32_t launch_mla_decode(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream) {
    const MlaShape d = mla_shape(a);
    MlaParams p{};
    p.q = static_cast<const uint16_t*>(a.q);
    p.q_st = a.q_stride_token;
    p.q_sh = a.q_stride_head;
    p.kv = static_cast<const uint16_t*>(a.k_pool);
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
    p.order = d.plan && d.n_units > 0 ? reinterpret_cast<int32_t*>(ws) : nullptr;
    p.ws_rec = d.n_chunks > 1 ? reinterpret_cast<float*>(ws + (d.plan ? align256(4 * d.n_units) : 0)) : nullptr;
    p.rec_floats = d.rec_floats;
    p.B = a.num_rows;
    p.T = a.num_tokens;
    p.P = a.num_partners;
    p.stripe_begin = a.stripe_begin;
    p.S = a.stripe_count;
    p.Hq = a.num_q_heads;
    p.max_pages = a.max_pages;
    p.page_size = a.page_size;
    p.max_row_tokens = std::max(1, a.max_row_tokens);
    p.n_chunks = int32_t(d.n_chunks);
    p.chunk_tokens = int32_t(d.chunk_tokens);
    p.n_units = int32_t(d.n_units);
    p.pad_tokens_per_block = 4;
    p.pad_blocks = (a.num_tokens + 3) / 4;
    p.head_groups = int32_t(d.head_groups);
    p.work_blocks = int32_t(d.work_blocks);
    p.scale_log2 = a.scale * kLog2e;

    if (p.order) {
        hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(1024), 0, stream, p);
        if (int32_t st = check_launch("cp_paged_attn_partial (MLA plan)")) return st;
    }
    const int64_t blocks = d.work_blocks + p.pad_blocks;
    if (blocks > 0) {
        const dim3 grid{uint32_t(blocks), 1, 1};
        switch (d.nw) {
            case 1: hipLaunchKernelGGL(mla_decode_kernel<1>, grid, dim3(64), 0, stream, p); break;
            case 2: hipLaunchKernelGGL(mla_decode_kernel<2>, grid, dim3(128), 0, stream, p); break;
            default: hipLaunchKernelGGL(mla_decode_kernel<4>, grid, dim3(256), 0, stream, p); break;
        }
        if (int32_t st = check_launch("cp_paged_attn_partial (MLA decode)")) return st;
    }
    if (d.n_chunks > 1 && d.n_items > 0) {
        hipLaunchKernelGGL(mla_chunk_merge_kernel, dim3(uint32_t(d.n_items * (a.num_q_heads / 2))), dim3(256), 0,
                           stream, p);
        return check_launch("cp_paged_attn_partial (MLA chunk merge)");
    }
    return CPATTN_OK;
}

}  // namespace cpattn
