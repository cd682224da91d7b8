// bf16 GQA per-stripe paged partial for head_dim = head_dim_v = 128, built for gfx950 MFMA.
//
// What it computes is the partial of one partner: attention of a row's queries over the context positions that
// partner holds, returned as (out, natural-log lse) (mstar PR #1124, "Context / Sequence Parallel 1/5", PR description;
// context attention over the paged cache in the vLLM compare view "[Core] Add explicit layer parallel plans",
// FlashAttentionImpl._forward_with_dcp, which also splits the key range of one call into several pieces).
//
// Work decomposition. A work item is (row b, stripe s, kv head g, tile of 16 query rows, chunk of the stripe's local
// tokens); one 64-lane wave runs it. Query rows of a kv head are (token, head-in-group) pairs, so a decode step with
// G = 4 fills 4 rows of the 16 and a multi-token row fills more. Fixed-size chunks keep every wave busy for about the
// same time whatever the spread of context lengths. An item whose stripe fits in one chunk writes the stripe partial
// directly; otherwise each chunk writes its unnormalised partial (o, running max, running sum) to the workspace and a
// second small kernel merges the chunks of each item exactly. The kernel boundary orders the two, so no device-scope
// fence is needed (such fences write back and invalidate a whole XCD L2, which costs far more than the extra launch).
// Items are ordered kv head fastest, so the heads of one page are read at about the same time and, with the
// hardware's round-robin of blocks over the 8 XCDs, each XCD receives an equal share of every row.
//
// Per step of 16 local tokens:
//   * scores S^T[token][row] = K . Q^T with four v_mfma_f32_16x16x32_bf16 (k = 32 head dims each). Lane l feeds token
//     l%16's dims [32i + 8(l/16), +8) as the A operand and query row l%16's same dims as the B operand, so each of the
//     four 16-byte K loads reads 16 whole 64-byte segments. The result leaves lane l with rows l%16 for tokens
//     4(l/16)+0..3, exactly the A-operand layout of the value product.
//   * online softmax in log2 units with a lazily moved running max (it moves only when a block maximum exceeds it by
//     more than 8, so most steps skip the rescale; probabilities stay <= 256 and fp32 sums stay exact enough).
//   * out += P . V with v_mfma_f32_16x16x16_bf16 (P split into a bf16 high part and a bf16 residual). Lane l loads tokens 4(l/16)+e, dims [8(l%16), +8): 16 lanes
//     read a whole 256-byte row, fully coalesced. Output tile n column j is taken to be head dim 8j + n, so the B
//     operand of tile n is element n of the lane's four token vectors: four 16-bit halves regrouped with two byte
//     permutes, no LDS round trip.
#include "launch.h"

#include <cstdlib>
#include <string>
#include <type_traits>

namespace cpattn {



struct DecodeParams {
    const uint16_t* q;
    int64_t q_st, q_sh;
    const uint16_t* kp;
    const uint16_t* vp;
    PoolGeom geo;
    const int32_t* q_row_start;
    const int32_t* ctx_len;
    const int32_t* bt;
    int64_t bt_stride;
    float* out;
    int64_t o_ss, o_st, o_sh;
    float* lse;
    int64_t l_ss, l_st;
    float* ws_rec;
    int32_t* ws_rowpref;          // persistent schedule: step offset of every row (B + 1 entries, the last the total)
    int32_t B, T, P, stripe_begin, S, Hq, Hkv, G;
    int32_t max_pages, page_size, max_row_tokens;
    int32_t ctx_cap;              // context lengths are clamped to min(max_pages * page_size, max_ctx_len)
    int32_t n_qtiles, n_chunks, chunk_steps;
    int32_t total_items, pad_blocks, pad_tokens_per_block;
    int32_t rec_rows;
    int32_t num_tiles, nwaves;    // persistent schedule
    float scale_log2;             // softmax scale (times the key descale for fp8 pools) in log2 units
    float v_scale;                // value descale of fp8 pools, else 1 (applied where output rows are written)
    int32_t pad_lse_only;         // CPATTN_FLAG_PAD_LSE_ONLY: padding tokens get their lse only
    void* m_out;                  // fused finish: merged output [T, Hq, 128] (fp32 or bf16), its lse (nullable)
    int64_t m_st, m_sh;
    float* m_lse;
    int64_t m_lst;
};

// s_waitcnt with vmcnt = 0 and the other counters at their maximum (gfx9 encoding: vmcnt bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]).
__device__ __forceinline__ void wait_all_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// K/V loads. A call reads each context K/V byte once, so the loads carry the nontemporal hint (CPATTN_KV_NONTEMPORAL,
// default on). On a plain sequential 2 GiB read the hinted loads streamed at ~7.0 TB/s against ~6.3 TB/s for
// default-policy loads on the same device.
#ifndef CPATTN_KV_NONTEMPORAL
#define CPATTN_KV_NONTEMPORAL 1
#endif
template <typename V>
__device__ __forceinline__ V load_kv(const void* p) {
    if (CPATTN_KV_NONTEMPORAL) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
    return *reinterpret_cast<const V*>(p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Load mapping. Instruction e of a step reads, for K and V alike, the step tokens 4e + l/16 at head dims
// [8*(l%16), +8): sixteen lanes cover one 256-byte row and the 64 lanes four consecutive tokens, i.e. one contiguous
// stretch of a page (a whole page of one head when page_size / P = 4). Fragmenting an instruction over several pages
// costs a large share of HBM bandwidth, so each instruction stays inside one page wherever the page allows. K and V
// pools share their layout, so one set of offsets serves both.
//
// Token order inside a step. The value product contracts over k = 4*(l/16) + e, which this mapping ties to step token
// 4e + l/16. Score row m of the MFMA is therefore given token sigma(m) = 4(m mod 4) + m/4, which puts the probability
// of token 4e + l/16 exactly where the value operand expects it.
//
// Addressing. When a physical page holds four or more slots, the four tokens of an instruction share one page, so its
// page id is the same for the whole wave: it is read from the block table with a scalar load, and the page base is
// formed on the scalar unit; each lane only adds its fixed offset (slot l/16, dims 8*(l%16)). Smaller pages pick the
// lane's page among two or four such bases. Page indices past the stripe's last page are clamped to it (the data of
// those tokens is discarded), and block-table entries outside [0, num_pages) read page 0.
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;

struct StepBase {
    int64_t base[4];   // element offset of instruction e's page for this lane (pool-relative)
};

template <int PPMODE>   // 2: pp >= 4, 1: pp == 2, 0: pp == 1
__device__ __forceinline__ void step_bases(StepBase& sb, const_i32_ptr bt_row, int32_t jb, int32_t last_pidx,
                                           int32_t c4, int64_t base_rg, const PoolGeom& geo) {
    if (PPMODE == 2) {
        // The step's 16 tokens lie on pages p0 .. p0 + 3 at most (pp >= 4). Away from the end of the row the four
        // block-table entries are read together (one scalar load, one wait); at the end each index is clamped.
        const int32_t p0 = jb >> geo.pp_shift;
        int32_t pg[4];
        if (p0 + 3 <= last_pidx) {
#pragma unroll
            for (int q = 0; q < 4; ++q) pg[q] = bt_row[p0 + q];
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) pg[q] = bt_row[min(p0 + q, last_pidx)];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int32_t j = jb + 4 * e;                  // first token of instruction e (a multiple of 4)
            const int32_t q = (j >> geo.pp_shift) - p0;
            int32_t page = q == 0 ? pg[0] : q == 1 ? pg[1] : q == 2 ? pg[2] : pg[3];
            page = (page >= 0 && page < geo.num_pages) ? page : 0;
            sb.base[e] = base_rg + int64_t(page) * geo.s_page + int64_t(j & (geo.pp - 1)) * geo.s_slot;
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int32_t j = jb + 4 * e;                      // first token of instruction e (a multiple of 4)
        {
            const int32_t n = PPMODE == 1 ? 2 : 4;            // pages touched by the instruction
            int64_t cand[4];
#pragma unroll
            for (int q = 0; q < n; ++q) {
                const int32_t pidx = min((j >> geo.pp_shift) + q, last_pidx);
                int32_t page = bt_row[pidx];
                page = (page >= 0 && page < geo.num_pages) ? page : 0;
                cand[q] = base_rg + int64_t(page) * geo.s_page;
            }
            sb.base[e] = PPMODE == 1 ? (c4 >= 2 ? cand[1] : cand[0])
                                     : (c4 == 0 ? cand[0] : c4 == 1 ? cand[1] : c4 == 2 ? cand[2] : cand[3]);
        }
    }
}

struct StepData {
    u32x4_t k[4];      // step token 4e + l/16, dims [8*(l%16), +8)
    u32x4_t v[4];
};

__device__ __forceinline__ void step_load(StepData& d, const uint16_t* __restrict__ kp,
                                          const uint16_t* __restrict__ vp, const StepBase& sb, uint32_t lane_off) {
#pragma unroll
    for (int e = 0; e < 4; ++e) d.k[e] = load_kv<u32x4_t>(kp + sb.base[e] + lane_off);
#pragma unroll
    for (int e = 0; e < 4; ++e) d.v[e] = load_kv<u32x4_t>(vp + sb.base[e] + lane_off);
}

// fp8 pools: the same lanes and dims, 8 one-byte E4M3 codes per lane and instruction. The codes stay packed while the
// step is in flight (half the registers of a bf16 step) and are widened to bf16 only when the step is computed.
struct StepData8 {
    u32x2_t k[4];
    u32x2_t v[4];
};

__device__ __forceinline__ void step_load(StepData8& d, const uint16_t* __restrict__ kp,
                                          const uint16_t* __restrict__ vp, const StepBase& sb, uint32_t lane_off) {
    const uint8_t* k8 = reinterpret_cast<const uint8_t*>(kp);
    const uint8_t* v8 = reinterpret_cast<const uint8_t*>(vp);
#pragma unroll
    for (int e = 0; e < 4; ++e) d.k[e] = load_kv<u32x2_t>(k8 + sb.base[e] + lane_off);
#pragma unroll
    for (int e = 0; e < 4; ++e) d.v[e] = load_kv<u32x2_t>(v8 + sb.base[e] + lane_off);
}

// Eight E4M3 codes (bytes 0..7) to eight bf16 in the same order. E4M3 values are exact in bf16, and the gfx950
// conversion decodes every code exactly (measured over all 256 codes); the descales are applied in fp32 elsewhere.
__device__ __forceinline__ u32x4_t widen_fp8(u32x2_t c) {
    const auto w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false);
    const auto w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true);
    const auto w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false);
    const auto w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true);
    return (u32x4_t){__builtin_bit_cast(uint32_t, w0), __builtin_bit_cast(uint32_t, w1),
                     __builtin_bit_cast(uint32_t, w2), __builtin_bit_cast(uint32_t, w3)};
}

__device__ __forceinline__ const StepData& widen(const StepData& d) { return d; }
__device__ __forceinline__ StepData widen(const StepData8& d) {
    StepData w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        w.k[e] = widen_fp8(d.k[e]);
        w.v[e] = widen_fp8(d.v[e]);
    }
    return w;
}

template <bool KV8>
using StepBuf = typename std::conditional<KV8, StepData8, StepData>::type;

struct SoftmaxState {
    f32x4_t o[8];      // o[n][ii]: query row 4*(l/16)+ii, head dim 8*(l%16)+n (unnormalised)
    float m;           // running max (log2 units) of query row l%16
    float l;           // this lane's share of the running sum of query row l%16
};

// LDS slot (16-byte units) of step token t, head-dim block j, in the K re-layout buffer. The XOR with t spreads both
// the row-wise writes and the column-wise MFMA-operand reads over all bank groups.
__device__ __forceinline__ int kx_index(int t, int j) { return (t & 3) * 64 + (t >> 2) * 16 + (j ^ t); }

__device__ __forceinline__ int sigma(int m) { return 4 * (m & 3) + (m >> 2); }

__device__ __forceinline__ void step_compute(SoftmaxState& st, const StepData& d, const bf16x8_t (&qop)[4],
                                             u32x4_t* __restrict__ kx, int32_t jb, int32_t j1, int32_t n16,
                                             int32_t c4, float scale_log2) {
    // K from load layout (token per lane group, dims across lanes) to A-operand layout (token sigma(l%16) per lane,
    // dim block per lane group) through LDS. LDS operations of one wave complete in order: no barrier is needed.
#pragma unroll
    for (int e = 0; e < 4; ++e) kx[kx_index(4 * e + c4, n16)] = d.k[e];
    u32x4_t kop[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kop[i] = kx[kx_index(sigma(n16), 4 * i + c4)];

    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[i]), qop[i], sacc, 0, 0, 0);

    const bool tail = jb + 16 > j1;  // wave-uniform
    float sv[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        sv[ii] = sacc[ii] * scale_log2;          // score of step token 4*ii + l/16
        if (tail && jb + 4 * ii + c4 >= j1) sv[ii] = neg_inf();
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > st.m + 8.0f)) {
        const float m_new = fmaxf(st.m, mx);
        const float alpha = exp2f(st.m - m_new);   // 0 on the first step (m = -inf)
        st.l *= alpha;
        st.m = m_new;
        float a_o[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) a_o[ii] = __shfl(alpha, 4 * c4 + ii);
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) st.o[n][ii] *= a_o[ii];
    }
    float pv[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) pv[ii] = __builtin_amdgcn_exp2f(sv[ii] - st.m);
    st.l += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    // P enters the value product as a bf16 pair hi + lo (hi = bf16(p), lo = bf16(p - hi)): about 16 significant bits,
    // so a peaked softmax over a few tokens keeps fp32-level accuracy. The second MFMA per tile is cheap next to the
    // memory time of a step.
    const u32x2_t pw = {pack2_bf16(pv[0], pv[1]), pack2_bf16(pv[2], pv[3])};
    const s16x4_t pop = __builtin_bit_cast(s16x4_t, pw);
    float pr[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const uint32_t w = pw[ii >> 1];
        pr[ii] = pv[ii] - __uint_as_float((ii & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    const u32x2_t pwl = {pack2_bf16(pr[0], pr[1]), pack2_bf16(pr[2], pr[3])};
    const s16x4_t pop_lo = __builtin_bit_cast(s16x4_t, pwl);

    u32x4_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = d.v[e];
        if (tail && jb + 4 * e + c4 >= j1) v[e] = (u32x4_t){0u, 0u, 0u, 0u};   // select, never 0 * NaN
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int dw = n >> 1;
        const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(v[1][dw], v[0][dw], sel);
        const uint32_t hi = __builtin_amdgcn_perm(v[3][dw], v[2][dw], sel);
        const s16x4_t vop = __builtin_bit_cast(s16x4_t, (u32x2_t){lo, hi});
        st.o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pop, vop, st.o[n], 0, 0, 0);
        st.o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pop_lo, vop, st.o[n], 0, 0, 0);
    }
}

__device__ __forceinline__ void write_row(const DecodeParams& p, int32_t s, int32_t tok0, int32_t row0, int32_t g,
                                          int32_t row, int32_t n16, const float (&vals)[8]) {
    const int32_t rho = row0 + row;
    const int32_t t = tok0 + rho / p.G;
    const int32_t h = g * p.G + rho % p.G;
    float* o = p.out + s * p.o_ss + int64_t(t) * p.o_st + int64_t(h) * p.o_sh + 8 * n16;
    const float c = p.v_scale;
    *reinterpret_cast<f32x4_t*>(o) = (f32x4_t){vals[0] * c, vals[1] * c, vals[2] * c, vals[3] * c};
    *reinterpret_cast<f32x4_t*>(o + 4) = (f32x4_t){vals[4] * c, vals[5] * c, vals[6] * c, vals[7] * c};
}

__device__ __forceinline__ void write_lse(const DecodeParams& p, int32_t s, int32_t tok0, int32_t row0, int32_t g,
                                          int32_t row, float m_log2, float l) {
    const int32_t rho = row0 + row;
    const int32_t t = tok0 + rho / p.G;
    const int32_t h = g * p.G + rho % p.G;
    p.lse[s * p.l_ss + int64_t(t) * p.l_st + h] = l > 0.f ? (m_log2 + log2f(l)) * kLn2 : neg_inf();
}

template <int DEPTH, int PPMODE, bool KV8>
__global__ __launch_bounds__(64) void gqa_decode_bf16_kernel(const DecodeParams p) {
    __shared__ u32x4_t s_kx[256];
    const int lane = threadIdx.x;
    // The hardware hands block i to XCD i mod 8. With the kv head fastest in the item order and Hkv a multiple of 8,
    // every XCD gets the same heads of every row: equal work per XCD whatever the spread of row lengths.
    const int32_t logical = blockIdx.x;

    if (logical >= p.total_items) {               // padding-token fill role
        const int32_t k = logical - p.total_items;
        if (k >= p.pad_blocks) return;
        const int32_t first = min(max(p.q_row_start[p.B], 0), p.T);
        const int32_t t0 = max(k * p.pad_tokens_per_block, first);
        const int32_t t1 = min((k + 1) * p.pad_tokens_per_block, p.T);
        if (t0 < t1)
            fill_padding(p.out, p.o_ss, p.o_st, p.o_sh, p.lse, p.l_ss, p.l_st, p.S, p.Hq, 128, t0, t1, lane, 64,
                         p.pad_lse_only);
        return;
    }

    // Item order (kv head fastest, then chunk, tile, stripe, row): the heads of one page run side by side.
    int32_t item = logical;
    const int32_t g = item % p.Hkv;
    item /= p.Hkv;
    const int32_t c = item % p.n_chunks;
    item /= p.n_chunks;
    const int32_t qt = item % p.n_qtiles;
    item /= p.n_qtiles;
    const int32_t s = item % p.S;
    const int32_t b = item / p.S;

    const int32_t tok0 = min(max(p.q_row_start[b], 0), p.T);
    const int32_t tok1 = min(max(p.q_row_start[b + 1], tok0), p.T);
    if (g == 0 && c == 0 && qt == p.n_qtiles - 1)
        fill_excess_tokens(p.out + s * p.o_ss, p.o_st, p.o_sh, p.lse + s * p.l_ss, p.l_st, tok0, tok1, p.max_row_tokens,
                           p.Hq, 128, lane, 64, p.pad_lse_only);
    const int32_t ntok = min(tok1 - tok0, p.max_row_tokens);
    const int32_t nrows = ntok * p.G;
    const int32_t row0 = qt * 16;
    if (row0 >= nrows) return;
    const int32_t tile_rows = min(16, nrows - row0);

    const int32_t r = p.stripe_begin + s;
    const int32_t L = min(max(p.ctx_len[b], 0), p.ctx_cap);
    const int32_t Lr = stripe_length(L, r, p.P, p.geo.interleave);
    const int32_t CH = p.chunk_steps * 16;
    const int32_t nch = (Lr + CH - 1) / CH;
    if (c >= max(nch, 1)) return;
    const int32_t j0 = c * CH;
    const int32_t j1 = min(j0 + CH, Lr);

    const int32_t n16 = lane & 15;
    const int32_t c4 = lane >> 4;

    // Query operand: row n16 of the tile, dims [32i + 8*c4, +8).
    bf16x8_t qop[4];
    {
        const int32_t rho = row0 + n16;
        if (rho < nrows) {
            const uint16_t* qp = p.q + int64_t(tok0 + rho / p.G) * p.q_st + int64_t(g * p.G + rho % p.G) * p.q_sh + 8 * c4;
#pragma unroll
            for (int i = 0; i < 4; ++i) qop[i] = as_bf16x8(load16(qp + 32 * i));
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) qop[i] = as_bf16x8((u32x4_t){0u, 0u, 0u, 0u});
        }
    }

    // Retire the query loads here, before the first prefetch is issued: the wait-count pass cannot tell, inside the
    // loop, that these older loads finished, and would otherwise drain every outstanding load (the prefetched steps
    // included) before the first use of the query operand in each iteration.
    wait_all_vmem();
    const const_i32_ptr bt_row = (const_i32_ptr)(p.bt + int64_t(b) * p.bt_stride);
    const int32_t last_pidx = Lr > 0 ? (Lr - 1) >> p.geo.pp_shift : 0;
    // Lane offset inside instruction e's page run: slot within the page plus the lane's dim block.
    const int32_t lane_slot = PPMODE == 2 ? c4 : (PPMODE == 1 ? (c4 & 1) : 0);
    const uint32_t lane_off = uint32_t(lane_slot * p.geo.s_slot + 8 * n16);

    SoftmaxState st;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    st.m = neg_inf();
    st.l = 0.f;

    // Ring of DEPTH register buffers: the loads of step k + DEPTH - 1 are in flight while step k is computed. Every
    // prefetch is issued unconditionally (a step past the end re-reads the chunk's last step, a cache hit), so the
    // number of loads in flight is the same on every path and each wait only retires the step about to be used.
    const int64_t base_rg = int64_t(r) * p.geo.s_stripe + int64_t(g) * p.geo.s_head;
    const int32_t nsteps = (j1 - j0 + 15) >> 4;
    const int32_t last = max(nsteps - 1, 0);
    StepBuf<KV8> buf[DEPTH];
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u) {
        StepBase sb;
        step_bases<PPMODE>(sb, bt_row, j0 + 16 * min(u, last), last_pidx, c4, base_rg, p.geo);
        step_load(buf[u], p.kp, p.vp, sb, lane_off);
    }
    for (int32_t it = 0; it < nsteps; it += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const int32_t k = it + u;
            {
                StepBase sb;
                step_bases<PPMODE>(sb, bt_row, j0 + 16 * min(k + DEPTH - 1, last), last_pidx, c4, base_rg, p.geo);
                step_load(buf[(u + DEPTH - 1) % DEPTH], p.kp, p.vp, sb, lane_off);
            }
            if (k < nsteps) step_compute(st, widen(buf[u]), qop, s_kx, j0 + 16 * k, j1, n16, c4, p.scale_log2);
        }
    }

    // Row sums: combine the four lane groups that share a query row.
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
    float l_o[4], m_o[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        l_o[ii] = __shfl(st.l, 4 * c4 + ii);
        m_o[ii] = __shfl(st.m, 4 * c4 + ii);
    }

    if (nch <= 1) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int32_t row = 4 * c4 + ii;
            if (row < tile_rows) {
                const float inv = l_o[ii] > 0.f ? 1.0f / l_o[ii] : 0.f;
                float vals[8];
#pragma unroll
                for (int n = 0; n < 8; ++n) vals[n] = st.o[n][ii] * inv;
                write_row(p, s, tok0, row0, g, row, n16, vals);
            }
        }
        if (c4 == 0 && n16 < tile_rows) write_lse(p, s, tok0, row0, g, n16, st.m, st.l);
        return;
    }

    // Several chunks: store this chunk's unnormalised record; gqa_decode_chunk_merge_kernel combines them.
    const int32_t RR = p.rec_rows;
    float* rec = p.ws_rec + int64_t(logical) * RR * 130;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const int32_t row = 4 * c4 + ii;
        if (row < tile_rows) {
            float* o = rec + row * 128 + 8 * n16;
            *reinterpret_cast<f32x4_t*>(o) = (f32x4_t){st.o[0][ii], st.o[1][ii], st.o[2][ii], st.o[3][ii]};
            *reinterpret_cast<f32x4_t*>(o + 4) = (f32x4_t){st.o[4][ii], st.o[5][ii], st.o[6][ii], st.o[7][ii]};
        }
    }
    if (c4 == 0 && n16 < tile_rows) {
        rec[RR * 128 + n16] = st.m;
        rec[RR * 128 + RR + n16] = st.l;
    }
}

// Exact merge of the chunk records of every item that needed more than one chunk: with M = max_c m_c,
// o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c and lse = (M + log2 sum_c 2^(m_c - M) l_c) ln 2.
// One wave per (row, stripe, query tile, kv head). Lane l handles query row 4*rg + l/16 (row groups rg of four rows)
// and head dims [8*(l%16), +8); the records of up to 16 chunks are loaded in one round.
__global__ __launch_bounds__(64) void gqa_decode_chunk_merge_kernel(const DecodeParams p) {
    const int lane = threadIdx.x;
    const int32_t triple = blockIdx.x;            // ((row * S + stripe) * n_qtiles + tile) * Hkv + kv head
    const int32_t g = triple % p.Hkv;
    int32_t item = triple / p.Hkv;
    const int32_t tile = item;
    const int32_t qt = item % p.n_qtiles;
    item /= p.n_qtiles;
    const int32_t s = item % p.S;
    const int32_t b = item / p.S;
    if (b >= p.B) return;
    const int32_t tok0 = min(max(p.q_row_start[b], 0), p.T);
    const int32_t tok1 = min(max(p.q_row_start[b + 1], tok0), p.T);
    const int32_t nrows = min(tok1 - tok0, p.max_row_tokens) * p.G;
    const int32_t row0 = qt * 16;
    if (row0 >= nrows) return;
    const int32_t tile_rows = min(16, nrows - row0);
    const int32_t L = min(max(p.ctx_len[b], 0), p.ctx_cap);
    const int32_t Lr = stripe_length(L, p.stripe_begin + s, p.P, p.geo.interleave);
    const int32_t CH = p.chunk_steps * 16;
    const int32_t nch = (Lr + CH - 1) / CH;
    if (nch <= 1) return;                       // written directly by the chunk kernel
    const int32_t d8 = lane & 15, rsub = lane >> 4;
    const int32_t RR = p.rec_rows;
    const int64_t rec_floats = int64_t(RR) * 130;
    // Chunk c of this item is record ((tile * n_chunks + c) * Hkv + g).
    const float* rec0 = p.ws_rec + (int64_t(tile) * p.n_chunks * p.Hkv + g) * rec_floats;
    const int64_t rec_step = int64_t(p.Hkv) * rec_floats;
    constexpr int kUnrolled = 16;

    for (int32_t rg = 0; 4 * rg < tile_rows; ++rg) {
        const int32_t row = 4 * rg + rsub;
        const bool active = row < tile_rows;
        const int32_t rrow = min(row, RR - 1);
        float M = neg_inf(), Lsum = 0.f;
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
        if (nch <= kUnrolled) {
            float mc[kUnrolled], lc[kUnrolled];
            f32x4_t o0[kUnrolled], o1[kUnrolled];
#pragma unroll
            for (int cc = 0; cc < kUnrolled; ++cc) {
                const bool live = active && cc < nch;
                const float* rc = rec0 + cc * rec_step;
                mc[cc] = live ? rc[RR * 128 + rrow] : neg_inf();
                lc[cc] = live ? rc[RR * 128 + RR + rrow] : 0.f;
                o0[cc] = live ? *reinterpret_cast<const f32x4_t*>(rc + rrow * 128 + 8 * d8) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
                o1[cc] = live ? *reinterpret_cast<const f32x4_t*>(rc + rrow * 128 + 8 * d8 + 4) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int cc = 0; cc < kUnrolled; ++cc) M = fmaxf(M, mc[cc]);
#pragma unroll
            for (int cc = 0; cc < kUnrolled; ++cc) {
                const float w = cc < nch ? exp2f(mc[cc] - M) : 0.f;
                Lsum += w * lc[cc];
                a0 += w * o0[cc];
                a1 += w * o1[cc];
            }
        } else {
            for (int32_t cc = 0; cc < nch; ++cc) M = fmaxf(M, rec0[cc * rec_step + RR * 128 + rrow]);
            for (int32_t cc = 0; cc < nch; ++cc) {
                const float* rc = rec0 + cc * rec_step;
                const float w = exp2f(rc[RR * 128 + rrow] - M);
                Lsum += w * rc[RR * 128 + RR + rrow];
                a0 += w * *reinterpret_cast<const f32x4_t*>(rc + rrow * 128 + 8 * d8);
                a1 += w * *reinterpret_cast<const f32x4_t*>(rc + rrow * 128 + 8 * d8 + 4);
            }
        }
        if (active) {
            const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
            const float vals[8] = {a0[0] * inv, a0[1] * inv, a0[2] * inv, a0[3] * inv,
                                   a1[0] * inv, a1[1] * inv, a1[2] * inv, a1[3] * inv};
            write_row(p, s, tok0, row0, g, row, d8, vals);
            if (d8 == 0) write_lse(p, s, tok0, row0, g, row, M, Lsum);
        }
    }
}

// ============================================================================================ persistent schedule
//
// The grid is exactly the resident wave slots. Work is the flattened space (kv head g, tile T, step) with g slowest;
// tile T = (row, stripe, query tile) has n_T = ceil(Lr / 16) steps when it holds query rows. Every wave takes an
// equal contiguous range of that space, so all waves stream for the same time whatever the row lengths, and none is
// spent launching or retiring blocks. A range crosses item boundaries: only its first and last segments can be part of
// an item, so each wave writes at most two records (slot 0: first segment, slot 1: last segment); items covered by a
// single wave are written directly. gqa_decode_fixup_kernel merges split items, writes tiles without context and the
// padding tokens.

// Steps of tile T (0 when the tile holds no query row). Per-lane T: vector loads.
// Steps of tile T from its row's q_row_start[b], q_row_start[b + 1] and ctx_len[b].
__device__ __forceinline__ int32_t tile_steps_of(const DecodeParams& p, int32_t T, int32_t qrs0, int32_t qrs1,
                                                 int32_t ctx) {
    const int32_t qt = T % p.n_qtiles;
    const int32_t s = (T / p.n_qtiles) % p.S;
    const int32_t tok0 = min(max(qrs0, 0), p.T);
    const int32_t tok1 = min(max(qrs1, tok0), p.T);
    const int32_t nrows = min(tok1 - tok0, p.max_row_tokens) * p.G;
    const int32_t L = min(max(ctx, 0), p.ctx_cap);
    const int32_t Lr = stripe_length(L, p.stripe_begin + s, p.P, p.geo.interleave);
    return qt * 16 < nrows ? (Lr + 15) >> 4 : 0;
}

__device__ __forceinline__ int32_t tile_steps(const DecodeParams& p, int32_t T) {
    const int32_t b = (T / p.n_qtiles) / p.S;
    return tile_steps_of(p, T, p.q_row_start[b], p.q_row_start[b + 1], p.ctx_len[b]);
}

struct Tile {
    int32_t b, s, qt, tok0, nrows, Lr, n_steps;
    int32_t q0, q1, cl;      // the row's q_row_start[b], q_row_start[b + 1] and ctx_len[b] as read
};

// Wave-uniform T: scalar loads through the constant address space.
__device__ __forceinline__ Tile load_tile(const DecodeParams& p, int32_t T) {
    const const_i32_ptr qrs = (const_i32_ptr)p.q_row_start;
    const const_i32_ptr cl = (const_i32_ptr)p.ctx_len;
    Tile tl;
    tl.qt = T % p.n_qtiles;
    const int32_t bs = T / p.n_qtiles;
    tl.s = bs % p.S;
    tl.b = bs / p.S;
    tl.q0 = qrs[tl.b];
    tl.q1 = qrs[tl.b + 1];
    tl.cl = cl[tl.b];
    tl.tok0 = min(max(tl.q0, 0), p.T);
    const int32_t tok1 = min(max(tl.q1, tl.tok0), p.T);
    tl.nrows = min(tok1 - tl.tok0, p.max_row_tokens) * p.G;
    const int32_t L = min(max(tl.cl, 0), p.ctx_cap);
    tl.Lr = stripe_length(L, p.stripe_begin + tl.s, p.P, p.geo.interleave);
    tl.n_steps = tl.qt * 16 < tl.nrows ? (tl.Lr + 15) >> 4 : 0;
    return tl;
}

// Steps of all tiles of a row (every stripe, every query tile holding rows) from its q_row_start pair and ctx_len;
// nq = its query tiles holding rows. Tiles of a row are ordered stripe-major, query tile minor.
__device__ __forceinline__ int32_t row_steps_of(const DecodeParams& p, int32_t qrs0, int32_t qrs1, int32_t ctx,
                                                int32_t& nq) {
    const int32_t tok0 = min(max(qrs0, 0), p.T);
    const int32_t tok1 = min(max(qrs1, tok0), p.T);
    const int32_t nrows = min(tok1 - tok0, p.max_row_tokens) * p.G;
    nq = (nrows + 15) >> 4;
    const int32_t L = min(max(ctx, 0), p.ctx_cap);
    int32_t steps = 0;
    for (int32_t s = 0; s < p.S; ++s) steps += (stripe_length(L, p.stripe_begin + s, p.P, p.geo.interleave) + 15) >> 4;
    return nq * steps;
}

// The tile of row b holding the row's step `off` (0 <= off < the row's steps); off becomes the step inside the tile.
__device__ __forceinline__ Tile tile_in_row(const DecodeParams& p, int32_t b, int32_t qrs0, int32_t qrs1, int32_t ctx,
                                            int32_t& off) {
    Tile tl;
    tl.b = b;
    tl.q0 = qrs0;
    tl.q1 = qrs1;
    tl.cl = ctx;
    tl.tok0 = min(max(qrs0, 0), p.T);
    const int32_t tok1 = min(max(qrs1, tl.tok0), p.T);
    tl.nrows = min(tok1 - tl.tok0, p.max_row_tokens) * p.G;
    const int32_t nq = (tl.nrows + 15) >> 4;
    const int32_t L = min(max(ctx, 0), p.ctx_cap);
    tl.s = 0;
    tl.Lr = 0;
    tl.n_steps = 0;
    tl.qt = 0;
    for (int32_t s = 0; s < p.S; ++s) {
        const int32_t Lr = stripe_length(L, p.stripe_begin + s, p.P, p.geo.interleave);
        const int32_t n = (Lr + 15) >> 4;
        if (off < nq * n) {
            tl.s = s;
            tl.Lr = Lr;
            tl.n_steps = n;
            tl.qt = off / n;
            off -= tl.qt * n;
            break;
        }
        off -= nq * n;
    }
    return tl;
}

// Step offset of every row (ws_rowpref[b], b <= B, the last entry the total), written by one wave of the persistent
// kernel for the kernels that run after it: the lanes hold consecutive row blocks with their exclusive offsets.
__device__ __forceinline__ void publish_row_prefix(const DecodeParams& p, int32_t r_lo, int32_t r_hi, int32_t excl,
                                                   int32_t total, int lane) {
    int32_t acc = excl;
    for (int32_t b = r_lo; b < r_hi; ++b) {
        p.ws_rowpref[b] = acc;
        int32_t nq;
        acc += row_steps_of(p, p.q_row_start[b], p.q_row_start[b + 1], p.ctx_len[b], nq);
    }
    if (lane == 0) p.ws_rowpref[p.B] = total;
}

// Step offset of tile (row b, stripe s, query tile qt) inside the step space of one kv head, from the published row
// offsets.
__device__ __forceinline__ int32_t tile_offset(const DecodeParams& p, int32_t b, int32_t s, int32_t qt, int32_t qrs0,
                                               int32_t qrs1, int32_t ctx) {
    int32_t nq;
    (void)row_steps_of(p, qrs0, qrs1, ctx, nq);
    const int32_t L = min(max(ctx, 0), p.ctx_cap);
    int32_t off = p.ws_rowpref[b];
    for (int32_t s2 = 0; s2 < s; ++s2) off += nq * ((stripe_length(L, p.stripe_begin + s2, p.P, p.geo.interleave) + 15) >> 4);
    return off + qt * ((stripe_length(L, p.stripe_begin + s, p.P, p.geo.interleave) + 15) >> 4);
}

struct ItemAddr {
    const int32_t* bt_row;
    int64_t base_rg;
    int32_t last_pidx;
};

__device__ __forceinline__ ItemAddr item_addr(const DecodeParams& p, const Tile& tl, int32_t g) {
    ItemAddr ia;
    ia.bt_row = p.bt + int64_t(tl.b) * p.bt_stride;
    ia.base_rg = int64_t(p.stripe_begin + tl.s) * p.geo.s_stripe + int64_t(g) * p.geo.s_head;
    ia.last_pidx = tl.Lr > 0 ? (tl.Lr - 1) >> p.geo.pp_shift : 0;
    return ia;
}

// Block-table entries of one step, fetched a step ahead: lane i < 16 holds entry min(pbase + i, last_pidx) of the
// item's row, pbase = (16 k) >> pp_shift, which covers every page the step's 16 tokens touch (pp >= 1). The fetch is a
// vector load issued before the K/V loads of the step before it; vector loads complete in order, so by the time those
// K/V loads have been waited for, the entries are in registers and the next issue does not wait on memory.
__device__ __forceinline__ int32_t fetch_step_pages(const ItemAddr& ia, int32_t k, int lane, const PoolGeom& geo) {
    const int32_t pbase = (16 * k) >> geo.pp_shift;
    return ia.bt_row[min(pbase + (lane & 15), ia.last_pidx)];
}

// Page of block-table slot q (0 <= q < 16, wave-uniform) of a fetched step; invalid ids read page 0.
__device__ __forceinline__ int32_t step_page(int32_t pv, int32_t q, const PoolGeom& geo) {
    const int32_t page = __builtin_amdgcn_readlane(pv, q);
    return (page >= 0 && page < geo.num_pages) ? page : 0;
}

// Issue step k's K/V loads with its block-table entries `pv` (fetched earlier), and fetch step k + 1's entries into
// `pv`. Step index, last page index and the block-table row are wave-uniform; they go through readfirstlane so that
// everything derived from them stays scalar.
template <int PPMODE, typename SD>
__device__ __forceinline__ void issue_step(SD& d, int32_t& pv, const DecodeParams& p, const ItemAddr& ia, int32_t k,
                                           int32_t c4, uint32_t lane_off, int lane) {
    const int32_t ku = __builtin_amdgcn_readfirstlane(k);
    const int32_t cur = pv;
    pv = fetch_step_pages(ia, ku + 1, lane, p.geo);          // first: the K/V loads below may stay in flight
    const int32_t jb = 16 * ku;
    const int32_t pbase = jb >> p.geo.pp_shift;
    StepBase sb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int32_t j = jb + 4 * e;                        // first token of instruction e
        const int32_t q0 = (j >> p.geo.pp_shift) - pbase;
        if (PPMODE == 2) {
            sb.base[e] = ia.base_rg + int64_t(step_page(cur, q0, p.geo)) * p.geo.s_page +
                         int64_t(j & (p.geo.pp - 1)) * p.geo.s_slot;
        } else if (PPMODE == 1) {
            const int64_t c0 = ia.base_rg + int64_t(step_page(cur, q0, p.geo)) * p.geo.s_page;
            const int64_t c1 = ia.base_rg + int64_t(step_page(cur, q0 + 1, p.geo)) * p.geo.s_page;
            sb.base[e] = c4 >= 2 ? c1 : c0;
        } else {
            int64_t c[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) c[q] = ia.base_rg + int64_t(step_page(cur, q0 + q, p.geo)) * p.geo.s_page;
            sb.base[e] = c4 == 0 ? c[0] : c4 == 1 ? c[1] : c4 == 2 ? c[2] : c[3];
        }
    }
    step_load(d, p.kp, p.vp, sb, lane_off);
}

// Query operand staged in LDS: slot i*64 + lane holds lane's dims [32i + 8*(l/16), +8) of query row l%16.
__device__ __forceinline__ void stage_query(u32x4_t* __restrict__ sq, const bf16x8_t (&qop)[4], int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sq[i * 64 + lane] = __builtin_bit_cast(u32x4_t, qop[i]);
}

__device__ __forceinline__ void read_query(bf16x8_t (&qop)[4], const u32x4_t* __restrict__ sq, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) qop[i] = as_bf16x8(sq[i * 64 + lane]);
}

__device__ __forceinline__ void load_query(bf16x8_t (&qop)[4], const DecodeParams& p, const Tile& tl, int32_t g,
                                           int32_t n16, int32_t c4) {
    const int32_t rho = tl.qt * 16 + n16;
    if (rho < tl.nrows) {
        const uint16_t* qp = p.q + int64_t(tl.tok0 + rho / p.G) * p.q_st + int64_t(g * p.G + rho % p.G) * p.q_sh + 8 * c4;
#pragma unroll
        for (int i = 0; i < 4; ++i) qop[i] = as_bf16x8(load16(qp + 32 * i));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) qop[i] = as_bf16x8((u32x4_t){0u, 0u, 0u, 0u});
    }
}

// s_waitcnt vmcnt(8) (other counters at their maximum): the 8 loads of the newest step may stay in flight.
__device__ __forceinline__ void wait_vmem_8() { __builtin_amdgcn_s_waitcnt(0x0F78); }

// Finish a segment: the normalised stripe partial when the segment is the whole item, else an unnormalised record.
__device__ __forceinline__ void segment_epilogue(const DecodeParams& p, const SoftmaxState& st, const Tile& tl,
                                                 int32_t g, int32_t n16, int32_t c4, float* rec) {
    float lsum = st.l;
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    float l_o[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) l_o[ii] = __shfl(lsum, 4 * c4 + ii);
    const int32_t row0 = tl.qt * 16;
    const int32_t tile_rows = min(16, tl.nrows - row0);
    if (rec == nullptr) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int32_t row = 4 * c4 + ii;
            if (row < tile_rows) {
                const float inv = l_o[ii] > 0.f ? 1.0f / l_o[ii] : 0.f;
                float vals[8];
#pragma unroll
                for (int n = 0; n < 8; ++n) vals[n] = st.o[n][ii] * inv;
                write_row(p, tl.s, tl.tok0, row0, g, row, n16, vals);
            }
        }
        if (c4 == 0 && n16 < tile_rows) write_lse(p, tl.s, tl.tok0, row0, g, n16, st.m, lsum);
    } else {
        const int32_t RR = p.rec_rows;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int32_t row = 4 * c4 + ii;
            if (row < tile_rows) {
                float* o = rec + row * 128 + 8 * n16;
                *reinterpret_cast<f32x4_t*>(o) = (f32x4_t){st.o[0][ii], st.o[1][ii], st.o[2][ii], st.o[3][ii]};
                *reinterpret_cast<f32x4_t*>(o + 4) = (f32x4_t){st.o[4][ii], st.o[5][ii], st.o[6][ii], st.o[7][ii]};
            }
        }
        if (c4 == 0 && n16 < tile_rows) {
            rec[RR * 128 + n16] = st.m;
            rec[RR * 128 + RR + n16] = lsum;        // the whole row's sum, not this lane group's share
        }
    }
}

// Exclusive prefix of a wave-wide per-lane value (lane 0 gets 0) and the total.
__device__ __forceinline__ int32_t wave_exclusive_scan(int32_t v, int lane, int32_t& total) {
    int32_t incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
    }
    total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    return incl - v;
}

// A value every lane holds identically, moved to a scalar register so everything derived from it stays scalar.
__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

template <int PPMODE, bool KV8>
__global__ __launch_bounds__(64, 2) void gqa_decode_persist_kernel(const DecodeParams p) {
    __shared__ u32x4_t s_kx[256];
    __shared__ u32x4_t s_q[2][256];
    const int lane = threadIdx.x;
    const int32_t w = blockIdx.x;
    const int32_t nw = gridDim.x;
    const int32_t n16 = lane & 15, c4 = lane >> 4;
    const int32_t NT = p.num_tiles;

    // Step counts of every row (all its stripes and query tiles; the tiles of a row are contiguous in the step space):
    // lane l sums rows [R l, R l + R), a wave scan gives the lanes' offsets. Four rows' loads are issued before any is
    // used, so R rows cost ceil(R / 4) memory round trips; the first four rows' values stay in registers, so that the
    // search for this wave's first tile below needs no further load when R <= 4 (up to 256 rows).
    const int32_t R = (p.B + 63) >> 6;
    const int32_t r_lo = min(lane * R, p.B), r_hi = min(r_lo + R, p.B);
    int32_t kq0[4] = {0, 0, 0, 0}, kq1[4] = {0, 0, 0, 0}, kcl[4] = {0, 0, 0, 0};
    int32_t my_sum = 0;
    for (int32_t b = r_lo; b < r_hi; b += 4) {
        int32_t qa[4], qb[4], cl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int32_t bb = min(b + u, r_hi - 1);
            qa[u] = p.q_row_start[bb];
            qb[u] = p.q_row_start[bb + 1];
            cl[u] = p.ctx_len[bb];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int32_t nq;
            my_sum += b + u < r_hi ? row_steps_of(p, qa[u], qb[u], cl[u], nq) : 0;
        }
        if (b == r_lo) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                kq0[u] = qa[u];
                kq1[u] = qb[u];
                kcl[u] = cl[u];
            }
        }
    }
    int32_t N = 0;
    const int32_t my_excl = wave_exclusive_scan(my_sum, lane, N);
    if (w == 0) publish_row_prefix(p, r_lo, r_hi, my_excl, N, lane);
    // The host keeps Hkv * N below 2^31 for this schedule, so the step-space arithmetic is 32-bit (64-bit divisions
    // are long software sequences).
    const uint32_t total = uint32_t(p.Hkv) * uint32_t(N);
    const uint32_t Q = (total + uint32_t(nw) - 1) / uint32_t(nw);
    const uint32_t start = uint32_t(w) * Q;
    if (start >= total) return;
    int64_t remaining = min(Q, total - start);
    int32_t g = int32_t(start / uint32_t(N));
    const int32_t pos = int32_t(start - int64_t(g) * N);

    // The row holding `pos`: first the lane, then the row among the lane's (from registers when R <= 4, else one row
    // per lane and one scan), then the tile inside the row by arithmetic.
    const uint64_t owner = __ballot(my_sum > 0 && pos >= my_excl && pos < my_excl + my_sum);
    const int32_t src = uniform(int32_t(__builtin_ctzll(owner)));
    const int32_t src_lo = uniform(__shfl(r_lo, src));
    int32_t off = pos - uniform(__shfl(my_excl, src));
    int32_t rb, rq0, rq1, rcl;
    if (R <= 4) {
        rb = src_lo;
        rq0 = uniform(__shfl(kq0[0], src));
        rq1 = uniform(__shfl(kq1[0], src));
        rcl = uniform(__shfl(kcl[0], src));
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            int32_t nq;
            const int32_t n = row_steps_of(p, rq0, rq1, rcl, nq);
            if (off < n) break;
            off -= n;
            ++rb;
            rq0 = uniform(__shfl(kq0[u + 1], src));
            rq1 = uniform(__shfl(kq1[u + 1], src));
            rcl = uniform(__shfl(kcl[u + 1], src));
        }
    } else {
        const int32_t src_hi = uniform(__shfl(r_hi, src));
        const int32_t bl = src_lo + lane;
        int32_t q0v = 0, q1v = 0, clv = 0, n = 0, nq;
        if (bl < src_hi) {
            q0v = p.q_row_start[bl];
            q1v = p.q_row_start[bl + 1];
            clv = p.ctx_len[bl];
            n = row_steps_of(p, q0v, q1v, clv, nq);
        }
        int32_t dummy;
        const int32_t ex = wave_exclusive_scan(n, lane, dummy);
        const uint64_t hit = __ballot(n > 0 && off >= ex && off < ex + n);
        const int32_t hl = uniform(int32_t(__builtin_ctzll(hit)));
        off -= uniform(__shfl(ex, hl));
        rb = src_lo + hl;
        rq0 = uniform(__shfl(q0v, hl));
        rq1 = uniform(__shfl(q1v, hl));
        rcl = uniform(__shfl(clv, hl));
    }
    Tile tl = tile_in_row(p, rb, rq0, rq1, rcl, off);
    int32_t T = (tl.b * p.S + tl.s) * p.n_qtiles + tl.qt;
    int32_t seg_begin = off;

    const int32_t lane_slot = PPMODE == 2 ? c4 : (PPMODE == 1 ? (c4 & 1) : 0);
    const uint32_t lane_off = uint32_t(lane_slot * p.geo.s_slot + 8 * n16);
    float* const rec_base = p.ws_rec + int64_t(w) * 2 * p.rec_rows * 130;

    ItemAddr ia = item_addr(p, tl, g);
    int32_t seg_end = int32_t(min<int64_t>(tl.n_steps, seg_begin + remaining));
    bool first_seg = true;
    int qbuf = 0;                                    // LDS query buffer of the current item
    StepBuf<KV8> da, db;
    int32_t pv;                                      // block-table entries of the next step to issue
    {
        bf16x8_t q0[4];
        load_query(q0, p, tl, g, n16, c4);
        pv = fetch_step_pages(ia, seg_begin, lane, p.geo);
        issue_step<PPMODE>(da, pv, p, ia, seg_begin, c4, lane_off, lane);
        wait_vmem_8();                               // the query is in; the first step may still be in flight
        stage_query(s_q[0], q0, lane);
    }

    for (;;) {
        SoftmaxState st;
#pragma unroll
        for (int n = 0; n < 8; ++n) st.o[n] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        st.m = neg_inf();
        st.l = 0.f;
        const u32x4_t* sq = s_q[qbuf];
        // Steady state: steps go in pairs, step k in da and step k + 1 in db, so a buffer is never copied (copying a
        // buffer whose loads are in flight makes the wave wait for every load). Loads are unconditional: a step past
        // the segment (the second of an odd segment's last pair) is loaded and not computed; its addresses stay inside
        // the row's pages.
        const int32_t last = seg_end - 1;
        int32_t k = seg_begin;
        for (;;) {
            bf16x8_t qop[4];
            issue_step<PPMODE>(db, pv, p, ia, k + 1, c4, lane_off, lane);
            read_query(qop, sq, lane);
            step_compute(st, widen(da), qop, s_kx, 16 * k, tl.Lr, n16, c4, p.scale_log2);
            if (k + 2 > last) break;                 // db holds step k + 1: the segment's last, or past it
            issue_step<PPMODE>(da, pv, p, ia, k + 2, c4, lane_off, lane);
            read_query(qop, sq, lane);
            step_compute(st, widen(db), qop, s_kx, 16 * (k + 1), tl.Lr, n16, c4, p.scale_log2);
            k += 2;
        }
        // Last step of the segment (in db): the next item's query and first step (into da) are issued before it is
        // computed.
        remaining -= seg_end - seg_begin;
        bool more = remaining > 0;
        Tile nt = tl;
        ItemAddr na = ia;
        int32_t ng = g;
        bf16x8_t qn[4];
        if (more) {
            int32_t nT = T;
            do {
                if (++nT == NT) {
                    nT = 0;
                    ++ng;
                }
                nt = load_tile(p, nT);
            } while (nt.n_steps == 0 && ng < p.Hkv);
            if (ng < p.Hkv) {
                T = nT;
                na = item_addr(p, nt, ng);
                load_query(qn, p, nt, ng, n16, c4);
                pv = fetch_step_pages(na, 0, lane, p.geo);   // the next item's first entries (once per item)
                issue_step<PPMODE>(da, pv, p, na, 0, c4, lane_off, lane);
            } else {
                more = false;                        // cannot happen while steps remain; never read past the heads
            }
        }
        if (k + 1 <= last) {
            bf16x8_t qop[4];
            read_query(qop, sq, lane);
            step_compute(st, widen(db), qop, s_kx, 16 * (k + 1), tl.Lr, n16, c4, p.scale_log2);
        }
        if (more) {
            wait_vmem_8();
            stage_query(s_q[qbuf ^ 1], qn, lane);
        }
        const bool whole = seg_begin == 0 && seg_end == tl.n_steps;
        segment_epilogue(p, st, tl, g, n16, c4, whole ? nullptr : rec_base + (first_seg ? 0 : p.rec_rows * 130));
        if (!more) break;
        tl = nt;
        ia = na;
        g = ng;
        qbuf ^= 1;                                   // the new segment's first step is in da
        seg_begin = 0;
        seg_end = int32_t(min<int64_t>(tl.n_steps, remaining));
        first_seg = false;
    }
}

// Merge the records of an item split over waves wA..wB (A: its first step in the step space, Q: steps per wave) for
// record row rrow and head dims [8 d8, +8): one online pass over the covering waves' records, four loaded together
// (an item split over two waves, the usual case, costs one memory round trip); M is the running maximum (log2 units),
// earlier sums are rescaled when it rises. Records hold finite maxima (every segment has at least one key); unused
// batch entries carry -inf and weigh 0.
__device__ __forceinline__ void merge_records(const DecodeParams& p, int64_t A, int64_t Q, int64_t wA, int64_t wB,
                                              int32_t rrow, int32_t d8, float& M, float& Lsum, f32x4_t& a0,
                                              f32x4_t& a1) {
    const int32_t RR = p.rec_rows;
    const int64_t rec_floats = int64_t(RR) * 130;
    M = neg_inf();
    Lsum = 0.f;
    a0 = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    a1 = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    for (int64_t w0 = wA; w0 <= wB; w0 += 4) {
        float mc[4], lc[4];
        f32x4_t o0[4], o1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t wv = min(w0 + u, wB);
            const float* rc = p.ws_rec + (wv * 2 + (wv * Q >= A ? 0 : 1)) * rec_floats;
            mc[u] = rc[RR * 128 + rrow];
            lc[u] = rc[RR * 128 + RR + rrow];
            o0[u] = *reinterpret_cast<const f32x4_t*>(rc + rrow * 128 + 8 * d8);
            o1[u] = *reinterpret_cast<const f32x4_t*>(rc + rrow * 128 + 8 * d8 + 4);
            if (w0 + u > wB) mc[u] = neg_inf();
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < 4; ++u) Mn = fmaxf(Mn, mc[u]);
        const float f = M == neg_inf() ? 0.f : exp2f(M - Mn);
        Lsum *= f;
        a0 *= f;
        a1 *= f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float wgt = mc[u] == neg_inf() ? 0.f : exp2f(mc[u] - Mn);
            Lsum += wgt * lc[u];
            a0 += wgt * o0[u];
            a1 += wgt * o1[u];
        }
        M = Mn;
    }
}

// The fix-up and finish kernels run one independent wave per item, kFinishWaves of them a workgroup: fewer, larger
// workgroups start sooner than one single-wave workgroup per item.
constexpr int kFinishWaves = 4;

// Items split over several waves are merged from their records; tiles with query rows but no context get (0, -inf);
// extra waves write padding tokens. One wave per (tile, kv head).
__global__ __launch_bounds__(64 * kFinishWaves) void gqa_decode_fixup_kernel(const DecodeParams p) {
    const int lane = threadIdx.x & 63;
    const int32_t idx = int32_t(blockIdx.x) * kFinishWaves + int32_t(threadIdx.x >> 6);
    const int32_t n_items = p.num_tiles * p.Hkv;
    if (idx >= n_items + p.pad_blocks) return;
    if (idx >= n_items) {
        const int32_t k = idx - n_items;
        const int32_t first = min(max(p.q_row_start[p.B], 0), p.T);
        const int32_t t0 = max(k * p.pad_tokens_per_block, first);
        const int32_t t1 = min((k + 1) * p.pad_tokens_per_block, p.T);
        if (t0 < t1)
            fill_padding(p.out, p.o_ss, p.o_st, p.o_sh, p.lse, p.l_ss, p.l_st, p.S, p.Hq, 128, t0, t1, lane, 64,
                         p.pad_lse_only);
        return;
    }
    const int32_t T = idx / p.Hkv;
    const int32_t g = idx % p.Hkv;
    const Tile tl = load_tile(p, T);
    if (g == 0 && tl.qt == p.n_qtiles - 1)
        fill_excess_tokens(p.out + tl.s * p.o_ss, p.o_st, p.o_sh, p.lse + tl.s * p.l_ss, p.l_st, tl.tok0,
                           min(max(tl.q1, tl.tok0), p.T), p.max_row_tokens, p.Hq, 128, lane, 64, p.pad_lse_only);
    const int32_t row0 = tl.qt * 16;
    if (row0 >= tl.nrows) return;
    const int32_t tile_rows = min(16, tl.nrows - row0);
    const int32_t d8 = lane & 15, rsub = lane >> 4;
    if (tl.n_steps == 0) {                           // no context in this stripe: (0, -inf)
        const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int32_t rg = 0; 4 * rg < tile_rows; ++rg) {
            const int32_t row = 4 * rg + rsub;
            if (row < tile_rows) {
                write_row(p, tl.s, tl.tok0, row0, g, row, d8, zero);
                if (d8 == 0) write_lse(p, tl.s, tl.tok0, row0, g, row, neg_inf(), 0.f);
            }
        }
        return;
    }
    const int32_t N = p.ws_rowpref[p.B];
    const uint32_t total = uint32_t(p.Hkv) * uint32_t(N);
    const uint32_t Q = (total + uint32_t(p.nwaves) - 1) / uint32_t(p.nwaves);
    const uint32_t A = uint32_t(g) * uint32_t(N) + uint32_t(tile_offset(p, tl.b, tl.s, tl.qt, tl.q0, tl.q1, tl.cl));
    const uint32_t Bend = A + uint32_t(tl.n_steps);
    const int64_t wA = A / Q, wB = (Bend - 1) / Q;
    if (wA == wB) return;                            // one wave covered it and wrote it
    for (int32_t rg = 0; 4 * rg < tile_rows; ++rg) {
        const int32_t row = 4 * rg + rsub;
        const bool active = row < tile_rows;
        float M, Lsum;
        f32x4_t a0, a1;
        merge_records(p, A, Q, wA, wB, min(row, p.rec_rows - 1), d8, M, Lsum, a0, a1);
        if (active) {
            const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
            const float vals[8] = {a0[0] * inv, a0[1] * inv, a0[2] * inv, a0[3] * inv,
                                   a1[0] * inv, a1[1] * inv, a1[2] * inv, a1[3] * inv};
            write_row(p, tl.s, tl.tok0, row0, g, row, d8, vals);
            if (d8 == 0) write_lse(p, tl.s, tl.tok0, row0, g, row, M, Lsum);
        }
    }
}

// Fused finish of the persistent schedule when the call also merges the stripes (cp_paged_attn_merged): one wave per
// (row, query tile, kv head) assembles every stripe's partial of its rows - read back from the partial buffer where
// one wave covered the item, merged from the records where several did, (0, -inf) where the stripe holds no context -
// and combines them with the exact LSE merge of cp_lse_merge (the same helper), writing the merged output and lse. It
// also writes the split items' and empty stripes' partials, so the partial buffer ends as after cp_paged_attn_partial.
// Extra blocks write padding tokens: (0, -inf) in every partial and in the merged output.
template <bool BF16OUT, int SMAX>
__global__ __launch_bounds__(64 * kFinishWaves) void gqa_decode_finish_kernel(const DecodeParams p) {
    const int lane = threadIdx.x & 63;
    const int32_t idx = int32_t(blockIdx.x) * kFinishWaves + int32_t(threadIdx.x >> 6);
    const int32_t n_items = p.B * p.n_qtiles * p.Hkv;
    if (idx >= n_items + p.pad_blocks) return;
    const int32_t d8 = lane & 15, rsub = lane >> 4;
    auto merged_row = [&](int32_t t, int32_t h, const f32x4_t (&acc)[2]) __attribute__((always_inline)) {
        const int64_t off = int64_t(t) * p.m_st + int64_t(h) * p.m_sh + 8 * d8;
        if (BF16OUT) {
            const u32x4_t b = {pack2_bf16(acc[0][0], acc[0][1]), pack2_bf16(acc[0][2], acc[0][3]),
                               pack2_bf16(acc[1][0], acc[1][1]), pack2_bf16(acc[1][2], acc[1][3])};
            *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.m_out) + off) = b;
        } else {
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.m_out) + off) = acc[0];
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.m_out) + off + 4) = acc[1];
        }
    };
    if (idx >= n_items) {
        const int32_t k = idx - n_items;
        const int32_t first = min(max(p.q_row_start[p.B], 0), p.T);
        const int32_t t0 = max(k * p.pad_tokens_per_block, first);
        const int32_t t1 = min((k + 1) * p.pad_tokens_per_block, p.T);
        if (t0 >= t1) return;
        fill_padding(p.out, p.o_ss, p.o_st, p.o_sh, p.lse, p.l_ss, p.l_st, p.S, p.Hq, 128, t0, t1, lane, 64,
                     p.pad_lse_only);
        const f32x4_t zero[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        for (int32_t t = t0; t < t1; ++t)
            for (int32_t h = rsub; h < p.Hq; h += 4) merged_row(t, h, zero);
        if (p.m_lse)
            for (int32_t t = t0; t < t1; ++t)
                for (int32_t h = lane; h < p.Hq; h += 64) p.m_lse[int64_t(t) * p.m_lst + h] = neg_inf();
        return;
    }
    const int32_t g = idx % p.Hkv;
    const int32_t qt = (idx / p.Hkv) % p.n_qtiles;
    const int32_t b = (idx / p.Hkv) / p.n_qtiles;
    // The row's offsets, length and step offset in one round trip (scalar loads, all issued before any is used).
    const const_i32_ptr qrs = (const_i32_ptr)p.q_row_start;
    const const_i32_ptr clp = (const_i32_ptr)p.ctx_len;
    const const_i32_ptr rp = (const_i32_ptr)p.ws_rowpref;
    const int32_t q0 = qrs[b], q1 = qrs[b + 1], cl = clp[b], rowpref = rp[b], N = rp[p.B];
    const int32_t tok0 = min(max(q0, 0), p.T);
    const int32_t tok1 = min(max(q1, tok0), p.T);
    if (g == 0 && qt == p.n_qtiles - 1 && tok0 + p.max_row_tokens < tok1) {   // tokens past the host bound: padding
        for (int32_t s = 0; s < p.S; ++s)
            fill_excess_tokens(p.out + s * p.o_ss, p.o_st, p.o_sh, p.lse + s * p.l_ss, p.l_st, tok0, tok1,
                               p.max_row_tokens, p.Hq, 128, lane, 64, p.pad_lse_only);
        const f32x4_t zero[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        for (int32_t t = tok0 + p.max_row_tokens; t < tok1; ++t) {
            for (int32_t h = rsub; h < p.Hq; h += 4) merged_row(t, h, zero);
            if (p.m_lse)
                for (int32_t h = lane; h < p.Hq; h += 64) p.m_lse[int64_t(t) * p.m_lst + h] = neg_inf();
        }
    }
    const int32_t nrows = min(tok1 - tok0, p.max_row_tokens) * p.G;
    const int32_t row0 = qt * 16;
    if (row0 >= nrows) return;
    const int32_t tile_rows = min(16, nrows - row0);
    const int32_t nq = (nrows + 15) >> 4;
    const int32_t L = min(max(cl, 0), p.ctx_cap);
    const uint32_t total = uint32_t(p.Hkv) * uint32_t(N);
    const uint32_t Q = (total + uint32_t(p.nwaves) - 1) / uint32_t(p.nwaves);
    // Per stripe: its steps n, the item's first step A in the step space and the covering waves wA..wB. All loads of a
    // row group (partials of items one wave covered, the first two records of split items) are issued before anything
    // is stored, so a wave waits for one memory round trip rather than one per stripe.
    int32_t n_s[SMAX];
    uint32_t A_s[SMAX], wA_s[SMAX], wB_s[SMAX];
    {
        uint32_t off = uint32_t(g) * uint32_t(N) + uint32_t(rowpref);
#pragma unroll
        for (int32_t s = 0; s < SMAX; ++s) {
            const int32_t n = s < p.S ? (stripe_length(L, p.stripe_begin + s, p.P, p.geo.interleave) + 15) >> 4 : 0;
            n_s[s] = n;
            A_s[s] = off + uint32_t(qt * n);
            off += uint32_t(nq * n);
            wA_s[s] = n > 0 ? A_s[s] / Q : 0;
            wB_s[s] = n > 0 ? (A_s[s] + uint32_t(n) - 1) / Q : 0;
        }
    }
    const int32_t RR = p.rec_rows;
    const int64_t rec_floats = int64_t(RR) * 130;
    for (int32_t rg = 0; 4 * rg < tile_rows; ++rg) {
        const int32_t row = 4 * rg + rsub;
        const bool active = row < tile_rows;
        const int32_t rho = row0 + min(row, tile_rows - 1);
        const int32_t t = tok0 + rho / p.G;
        const int32_t h = g * p.G + rho % p.G;
        const int32_t rrow = min(row, RR - 1);
        // Loads, all unconditional (to addresses inside the buffers) so that they issue together: the partial row the
        // persistent kernel wrote, and the first two records of the item's covering waves (most items are split over
        // two waves at most; more take the general record merge below). What the item needs is selected after.
        float ls[SMAX], m0[SMAX], l0[SMAX], m1[SMAX], l1[SMAX];
        f32x4_t os[SMAX][2], r0[SMAX][2], r1[SMAX][2];
#pragma unroll
        for (int32_t s = 0; s < SMAX; ++s) {
            const int32_t sc = min(s, p.S - 1);
            const float* o = p.out + sc * p.o_ss + int64_t(t) * p.o_st + int64_t(h) * p.o_sh + 8 * d8;
            const float* lp = p.lse + sc * p.l_ss + int64_t(t) * p.l_st + h;
            const int64_t wA = wA_s[s];                  // (64-bit for the record addresses)
            const int64_t wA1 = min(wA + 1, int64_t(p.nwaves) - 1);
            const float* rc0 = p.ws_rec + (wA * 2 + (wA_s[s] * Q >= A_s[s] ? 0 : 1)) * rec_floats;
            const float* rc1 = p.ws_rec + (wA1 * 2) * rec_floats;   // the second wave starts inside the item
            os[s][0] = *reinterpret_cast<const f32x4_t*>(o);
            os[s][1] = *reinterpret_cast<const f32x4_t*>(o + 4);
            ls[s] = *lp;
            m0[s] = rc0[RR * 128 + rrow];
            l0[s] = rc0[RR * 128 + RR + rrow];
            r0[s][0] = *reinterpret_cast<const f32x4_t*>(rc0 + rrow * 128 + 8 * d8);
            r0[s][1] = *reinterpret_cast<const f32x4_t*>(rc0 + rrow * 128 + 8 * d8 + 4);
            m1[s] = rc1[RR * 128 + rrow];
            l1[s] = rc1[RR * 128 + RR + rrow];
            r1[s][0] = *reinterpret_cast<const f32x4_t*>(rc1 + rrow * 128 + 8 * d8);
            r1[s][1] = *reinterpret_cast<const f32x4_t*>(rc1 + rrow * 128 + 8 * d8 + 4);
        }
#pragma unroll
        for (int32_t s = 0; s < SMAX; ++s) {
            if (s < p.S && n_s[s] > 0 && wA_s[s] == wB_s[s]) continue;    // the partial row as loaded
            os[s][0] = os[s][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};          // empty stripe (or past S): (0, -inf)
            ls[s] = neg_inf();
        }
        // Stripe partials of split items (the arithmetic of merge_records and of the partial writes), then stores.
#pragma unroll
        for (int32_t s = 0; s < SMAX; ++s) {
            if (n_s[s] == 0 || wA_s[s] == wB_s[s]) continue;
            float M, Lsum;
            f32x4_t a0, a1;
            if (wB_s[s] == wA_s[s] + 1) {
                // merge_records over two records: the first batch of its loop with entries 2, 3 at -inf
                M = fmaxf(fmaxf(neg_inf(), m0[s]), m1[s]);
                const float w0 = m0[s] == neg_inf() ? 0.f : exp2f(m0[s] - M);
                const float w1 = m1[s] == neg_inf() ? 0.f : exp2f(m1[s] - M);
                Lsum = 0.f;
                a0 = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                a1 = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                Lsum += w0 * l0[s];
                a0 += w0 * r0[s][0];
                a1 += w0 * r0[s][1];
                Lsum += w1 * l1[s];
                a0 += w1 * r1[s][0];
                a1 += w1 * r1[s][1];
            } else {
                merge_records(p, A_s[s], Q, wA_s[s], wB_s[s], rrow, d8, M, Lsum, a0, a1);
            }
            // The values write_row and write_lse store for this partial.
            const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
            const float c = p.v_scale;
            os[s][0] = (f32x4_t){(a0[0] * inv) * c, (a0[1] * inv) * c, (a0[2] * inv) * c, (a0[3] * inv) * c};
            os[s][1] = (f32x4_t){(a1[0] * inv) * c, (a1[1] * inv) * c, (a1[2] * inv) * c, (a1[3] * inv) * c};
            ls[s] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : neg_inf();
        }
        if (!active) continue;
#pragma unroll
        for (int32_t s = 0; s < SMAX; ++s) {
            if (s >= p.S || (n_s[s] > 0 && wA_s[s] == wB_s[s])) continue;   // written by the persistent kernel
            float* o = p.out + s * p.o_ss + int64_t(t) * p.o_st + int64_t(h) * p.o_sh + 8 * d8;
            *reinterpret_cast<f32x4_t*>(o) = os[s][0];
            *reinterpret_cast<f32x4_t*>(o + 4) = os[s][1];
            if (d8 == 0) p.lse[s * p.l_ss + int64_t(t) * p.l_st + h] = ls[s];
        }
        f32x4_t acc[2];
        const float lse = lse_merge_rows<SMAX, 2>(ls, os, acc);
        merged_row(t, h, acc);
        if (d8 == 0 && p.m_lse) p.m_lse[int64_t(t) * p.m_lst + h] = lse;
    }
}

// Steps (16 keys each) of one chunk of the fixed-split schedule: splits fall every 1024 keys of a stripe.
constexpr int32_t kChunkSteps = 64;

constexpr int64_t kMaxPersistWaves = 8192;
constexpr int64_t kMaxPersistTiles = 4096;
// Workspace of the persistent schedule: the row offsets (B + 1 int32, padded to 256 bytes), then two records per wave.
inline int64_t rowpref_bytes(const cp_paged_args& a) { return (int64_t(a.num_rows + 1) * 4 + 255) / 256 * 256; }

struct DecodeShape {
    int64_t n_qtiles, n_chunks, total_items, rec_rows, triples, num_tiles;
    bool persistent;
};

static DecodeShape decode_shape(const cp_paged_args& a) {
    DecodeShape d{};
    const int64_t G = a.num_q_heads / a.num_kv_heads;
    const int64_t rows = int64_t(a.max_row_tokens) * G;
    d.n_qtiles = std::max<int64_t>(1, (rows + 15) / 16);
    d.num_tiles = int64_t(a.num_rows) * a.stripe_count * d.n_qtiles;
    // The persistent schedule's step space (kv heads x tiles x 16-key steps) is addressed with 32-bit arithmetic.
    const int64_t max_steps = (max_stripe_length(a) + 15) / 16;
    d.persistent = !(a.flags & CPATTN_FLAG_FIXED_SPLITS) && d.num_tiles <= kMaxPersistTiles &&
                   int64_t(a.num_kv_heads) * d.num_tiles * max_steps + kMaxPersistWaves < (int64_t(1) << 31);
    const int64_t max_lr = max_stripe_length(a);
    const int64_t CH = int64_t(kChunkSteps) * 16;
    d.n_chunks = d.persistent ? 1 : std::max<int64_t>(1, (max_lr + CH - 1) / CH);
    d.triples = d.num_tiles * a.num_kv_heads;
    d.total_items = d.triples * d.n_chunks;
    const int64_t rr = std::min<int64_t>(16, rows);
    d.rec_rows = std::max<int64_t>(4, (rr + 3) / 4 * 4);
    return d;
}

bool decode_bf16_eligible(const cp_paged_args& a, const PoolGeom& geo) {
    if (a.kind != CPATTN_GQA || a.dtype != CPATTN_BF16 || a.head_dim != 128 || a.head_dim_v != 128) return false;
    if (geo.pp_shift < 0 || geo.pp > 256) return false;
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    if (!al16(a.q) || !al16(a.k_pool) || !al16(a.v_pool) || !al16(a.out)) return false;
    if ((a.q_stride_token | a.q_stride_head | a.kv_stride_stripe | a.kv_stride_page | a.kv_stride_slot |
         a.kv_stride_head) & 7)
        return false;
    if ((a.out_stride_stripe | a.out_stride_token | a.out_stride_head) & 3) return false;
    const DecodeShape d = decode_shape(a);
    if (d.total_items + (a.num_tokens + 3) / 4 + 8 > (int64_t(1) << 31) - 1) return false;
    return true;
}

int64_t decode_bf16_workspace_bytes(const cp_paged_args& a) {
    const DecodeShape d = decode_shape(a);
    if (d.persistent) return rowpref_bytes(a) + kMaxPersistWaves * 2 * d.rec_rows * 130 * 4;
    if (d.n_chunks <= 1) return 0;
    return d.total_items * d.rec_rows * 130 * 4;
}

// Resident one-wave blocks of the persistent kernel on this device (cached per device and kernel variant).
template <int PPMODE, bool KV8>
static int32_t persistent_waves() {
    static int32_t cache[64][1] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cache[dev][0] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gqa_decode_persist_kernel<PPMODE, KV8>, 64, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 8;
        cache[dev][0] = int32_t(std::min<int64_t>(int64_t(cus) * per_cu, kMaxPersistWaves));
    }
    return cache[dev][0];
}

// Workspace bytes a launch on the current device actually touches: the persistent schedule writes records for the
// waves it launches (the device's resident-wave count), not for the kMaxPersistWaves the shape-only query assumes.
int64_t decode_bf16_workspace_bytes_on_device(const cp_paged_args& a, const PoolGeom& geo) {
    const DecodeShape d = decode_shape(a);
    if (!d.persistent) return decode_bf16_workspace_bytes(a);
    const bool kv8 = a.kv_format == CPATTN_KV_FP8_E4M3;
    const int ppmode = geo.pp_shift >= 2 ? 2 : geo.pp_shift;
    int32_t nw;
    if (ppmode == 2) nw = kv8 ? persistent_waves<2, true>() : persistent_waves<2, false>();
    else if (ppmode == 1) nw = kv8 ? persistent_waves<1, true>() : persistent_waves<1, false>();
    else nw = kv8 ? persistent_waves<0, true>() : persistent_waves<0, false>();
    return rowpref_bytes(a) + int64_t(nw) * 2 * d.rec_rows * 130 * 4;
}

// The fused finish holds every stripe's rows in registers: up to 8 stripes (more run the partial and merge calls).
bool decode_bf16_fuses_merge(const cp_paged_args& a) { return decode_shape(a).persistent && a.stripe_count <= 8; }

int32_t launch_paged_decode_bf16(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream,
                                 const cp_merge_out* m) {
    const DecodeShape d = decode_shape(a);
    DecodeParams p{};
    p.q = static_cast<const uint16_t*>(a.q);
    p.q_st = a.q_stride_token;
    p.q_sh = a.q_stride_head;
    p.kp = static_cast<const uint16_t*>(a.k_pool);
    p.vp = static_cast<const uint16_t*>(a.v_pool);
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
    p.n_qtiles = int32_t(d.n_qtiles);
    p.n_chunks = int32_t(d.n_chunks);
    p.chunk_steps = kChunkSteps;
    p.total_items = int32_t(d.total_items);
    p.pad_tokens_per_block = 4;
    p.pad_blocks = (a.num_tokens + 3) / 4;
    p.rec_rows = int32_t(d.rec_rows);
    p.num_tiles = int32_t(d.num_tiles);
    const bool kv8 = a.kv_format == CPATTN_KV_FP8_E4M3;
    p.scale_log2 = a.scale * (kv8 ? a.k_descale : 1.0f) * kLog2e;
    p.v_scale = kv8 ? a.v_descale : 1.0f;
    p.pad_lse_only = (a.flags & CPATTN_FLAG_PAD_LSE_ONLY) ? 1 : 0;
    const int ppmode = geo.pp_shift >= 2 ? 2 : geo.pp_shift;

    if (d.persistent) {
        p.ws_rowpref = static_cast<int32_t*>(a.workspace);
        p.ws_rec = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + rowpref_bytes(a));
        if (d.num_tiles > 0) {
            auto launch = [&](auto pp, auto k8) {
                constexpr int PP = decltype(pp)::value;
                constexpr bool K8 = decltype(k8)::value;
                const int32_t nw = persistent_waves<PP, K8>();
                p.nwaves = nw;
                hipLaunchKernelGGL((gqa_decode_persist_kernel<PP, K8>), dim3(uint32_t(nw)), dim3(64), 0, stream, p);
            };
            using T8 = std::true_type;
            using F8 = std::false_type;
            if (ppmode == 2)
                kv8 ? launch(std::integral_constant<int, 2>{}, T8{}) : launch(std::integral_constant<int, 2>{}, F8{});
            else if (ppmode == 1)
                kv8 ? launch(std::integral_constant<int, 1>{}, T8{}) : launch(std::integral_constant<int, 1>{}, F8{});
            else
                kv8 ? launch(std::integral_constant<int, 0>{}, T8{}) : launch(std::integral_constant<int, 0>{}, F8{});
            if (int32_t st = check_launch("cp_paged_attn_partial (bf16 decode, persistent)")) return st;
        }
        if (m) {                                     // fix-up and stripe merge in one launch
            p.m_out = m->out;
            p.m_st = m->out_stride_token;
            p.m_sh = m->out_stride_head;
            p.m_lse = m->lse;
            p.m_lst = m->lse_stride_token;
            const int64_t waves = int64_t(a.num_rows) * d.n_qtiles * a.num_kv_heads + p.pad_blocks;
            if (waves == 0) return CPATTN_OK;
            const dim3 grid{uint32_t((waves + kFinishWaves - 1) / kFinishWaves), 1, 1};
            const dim3 block{64 * kFinishWaves, 1, 1};
            const bool bf = m->out_dtype == CPATTN_BF16;
            if (a.stripe_count <= 4) {
                if (bf) hipLaunchKernelGGL((gqa_decode_finish_kernel<true, 4>), grid, block, 0, stream, p);
                else hipLaunchKernelGGL((gqa_decode_finish_kernel<false, 4>), grid, block, 0, stream, p);
            } else {
                if (bf) hipLaunchKernelGGL((gqa_decode_finish_kernel<true, 8>), grid, block, 0, stream, p);
                else hipLaunchKernelGGL((gqa_decode_finish_kernel<false, 8>), grid, block, 0, stream, p);
            }
            return check_launch("cp_paged_attn_merged (finish)");
        }
        const int64_t fix_waves = d.num_tiles * a.num_kv_heads + p.pad_blocks;
        if (fix_waves > 0) {
            hipLaunchKernelGGL(gqa_decode_fixup_kernel, dim3(uint32_t((fix_waves + kFinishWaves - 1) / kFinishWaves)),
                               dim3(64 * kFinishWaves), 0, stream, p);
            return check_launch("cp_paged_attn_partial (fix-up)");
        }
        return CPATTN_OK;
    }

    if (d.n_chunks > 1) p.ws_rec = static_cast<float*>(a.workspace);
    const int64_t blocks = ((d.total_items + p.pad_blocks) + 7) / 8 * 8;
    if (blocks == 0) return CPATTN_OK;
    const dim3 grid{uint32_t(blocks), 1, 1};
    if (kv8) {   // fp8 pools: the two-buffer ring (a step of codes is half the registers of a bf16 step)
        switch (ppmode) {
            case 0: hipLaunchKernelGGL((gqa_decode_bf16_kernel<2, 0, true>), grid, dim3(64), 0, stream, p); break;
            case 1: hipLaunchKernelGGL((gqa_decode_bf16_kernel<2, 1, true>), grid, dim3(64), 0, stream, p); break;
            default: hipLaunchKernelGGL((gqa_decode_bf16_kernel<2, 2, true>), grid, dim3(64), 0, stream, p); break;
        }
    } else {     // bf16 pools: the same two-buffer ring (the next step's loads in flight while one is computed)
        switch (ppmode) {
            case 0: hipLaunchKernelGGL((gqa_decode_bf16_kernel<2, 0, false>), grid, dim3(64), 0, stream, p); break;
            case 1: hipLaunchKernelGGL((gqa_decode_bf16_kernel<2, 1, false>), grid, dim3(64), 0, stream, p); break;
            default: hipLaunchKernelGGL((gqa_decode_bf16_kernel<2, 2, false>), grid, dim3(64), 0, stream, p); break;
        }
    }
    if (int32_t st = check_launch("cp_paged_attn_partial (bf16 decode)")) return st;
    if (d.n_chunks > 1 && d.triples > 0) {
        hipLaunchKernelGGL(gqa_decode_chunk_merge_kernel, dim3(uint32_t(d.triples)), dim3(64), 0, stream, p);
        return check_launch("cp_paged_attn_partial (chunk merge)");
    }
    return CPATTN_OK;
}

}  // namespace cpattn
