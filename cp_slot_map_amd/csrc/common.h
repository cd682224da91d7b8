// Internal helpers shared by the cpattn kernels and the host entry points (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cpattn.h"

namespace cpattn {

// ------------------------------------------------------------------------------------------------ host side
// Record a message for cpattn_last_error() and return `code`.
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Turn the launch status of the kernels just enqueued into a cpattn status.
int32_t check_launch(const char* what);

inline int ilog2_exact(int64_t x) {  // log2(x) if x is a power of two, else -1
    if (x <= 0 || (x & (x - 1))) return -1;
    int s = 0;
    while ((int64_t(1) << s) < x) ++s;
    return s;
}

// ------------------------------------------------------------------------------------------------ device side
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Element loads as fp32 from either storage type.
__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const uint16_t* p) { return bf16_bits_to_f32(*p); }
// One OCP E4M3 code of an fp8 pool (measured on gfx950: the conversion decodes all 256 codes exactly, subnormals
// and NaN included).
__device__ __forceinline__ float load_f32(const uint8_t* p) { return __builtin_amdgcn_cvt_pk_f32_fp8(uint32_t(*p), false)[0]; }

// Round to nearest even, as the hardware pack instruction does (NaN stays NaN).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    bf16x2_t h = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint16_t to_bf16_bits(float x) { return uint16_t(pack2_bf16(x, 0.0f) & 0xffffu); }

// Geometry of one stripe pool set (all P stripes): strides in elements and the page-to-slot split.
struct PoolGeom {
    int64_t s_stripe, s_page, s_slot, s_head;
    int32_t pp;          // slots per physical page = page_size / P
    int32_t pp_shift;    // log2(pp) if pp is a power of two, else -1
    int32_t num_pages;   // valid page ids are [0, num_pages); others read page 0
    int32_t interleave;  // I >= 1: runs of I consecutive logical slots go to one partner (I = 1: slot s to s mod P)
};

// Element offset of local token i of stripe r (kv head g) inside the pool set.
//
// Placement with interleave I (I = 1 is the slot rule of the PR): logical slot s goes to partner floor(s / I) mod P at
// physical slot floor(s / (I P)) * I + s mod I. With I P dividing page_size, local token i of partner r is the row's
// context position t = floor(i / I) * I * P + r * I + i mod I; its slot page * page_size + t mod page_size lands on
// logical page block_table[t / page_size] = block_table[i / pp] at physical slot i mod pp of r's pool (pp = page_size
// / P, a multiple of I): each stripe is an ordinary paged cache of page size pp sharing the logical block table, for
// every I. Every kernel that reads the pool goes through this.
__device__ __forceinline__ int64_t stripe_token_offset(const int32_t* __restrict__ bt_row, int32_t i, int32_t r,
                                                       int32_t g, const PoolGeom& geo) {
    int32_t pidx, slot;
    if (geo.pp_shift >= 0) {
        pidx = i >> geo.pp_shift;
        slot = i & (geo.pp - 1);
    } else {
        pidx = i / geo.pp;
        slot = i - pidx * geo.pp;
    }
    int32_t page = bt_row[pidx];
    page = (page >= 0 && page < geo.num_pages) ? page : 0;
    return int64_t(r) * geo.s_stripe + int64_t(page) * geo.s_page + int64_t(slot) * geo.s_slot +
           int64_t(g) * geo.s_head;
}

// Same split for a page id already read from the block table (used where page ids are staged in LDS).
__device__ __forceinline__ int64_t page_slot_offset(int32_t page, int32_t slot, int32_t r, int32_t g,
                                                    const PoolGeom& geo) {
    page = (page >= 0 && page < geo.num_pages) ? page : 0;
    return int64_t(r) * geo.s_stripe + int64_t(page) * geo.s_page + int64_t(slot) * geo.s_slot +
           int64_t(g) * geo.s_head;
}

// Tokens partner r holds of a row with L context tokens: positions t < L with floor(t / I) mod P == r, i.e. I tokens
// of every full cycle of I P positions plus those of the last, partial cycle.
__host__ __device__ __forceinline__ int32_t stripe_length(int32_t L, int32_t r, int32_t P, int32_t I) {
    if (L <= 0) return 0;
    const int32_t IP = I * P;
    const int32_t full = L / IP;
    const int32_t rest = L - full * IP - r * I;
    return full * I + (rest < 0 ? 0 : rest > I ? I : rest);
}

// Partner and physical slot of logical slot s >= 0 under interleave I.
__device__ __forceinline__ void place_slot(int64_t s, int64_t P, int64_t I, int32_t& partner, int64_t& phys) {
    const int64_t run = s / I;
    const int64_t cycle = run / P;
    partner = int32_t(run - cycle * P);
    phys = cycle * I + (s - run * I);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

// The exact LSE merge of cp_lse_merge over NMAX partials of KV float4s each (entries past the real partials carry
// lse = -inf): M = max_i l_i, w_i = exp(l_i - M), out = sum_i (w_i / sum w) o_i, lse = M + log(sum w); a partial with
// l_i = -inf is selected out (its row is never multiplied), and all of them -inf give (0, -inf). Entries with l = -inf
// change neither sum, so the result is the same for any NMAX. Shared by the merge kernel and the fused decode finish,
// with explicit fused multiply-adds, so that both give the same bits.
template <int NMAX, int KV>
__device__ __forceinline__ float lse_merge_rows(const float (&l)[NMAX], const f32x4_t (&o)[NMAX][KV],
                                                f32x4_t (&acc)[KV]) {
    float M = neg_inf();
#pragma unroll
    for (int i = 0; i < NMAX; ++i) M = fmaxf(M, l[i]);
#pragma unroll
    for (int v = 0; v < KV; ++v) acc[v] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    if (M == neg_inf()) return neg_inf();
    float w[NMAX];
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        w[i] = l[i] == neg_inf() ? 0.f : expf(l[i] - M);
        tot += w[i];
    }
    const float inv = 1.0f / tot;
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        const float c = w[i] * inv;
#pragma unroll
        for (int v = 0; v < KV; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = __builtin_fmaf(c, o[i][v][e], acc[v][e]);
                acc[v][e] = w[i] != 0.f ? f : acc[v][e];
            }
    }
    return M + logf(tot);
}

// Write (0, -inf) for padding query tokens [t_begin, t_end) of S partials (Hq heads, Dv dims each).
// With lse_only (CPATTN_FLAG_PAD_LSE_ONLY) the out rows are left as they are.
__device__ __forceinline__ void fill_padding(float* out, int64_t o_ss, int64_t o_st, int64_t o_sh, float* lse,
                                             int64_t l_ss, int64_t l_st, int32_t S, int32_t Hq, int32_t Dv,
                                             int32_t t_begin, int32_t t_end, int lane, int nlanes,
                                             bool lse_only = false) {
    for (int32_t t = t_begin; t < t_end; ++t) {
        for (int32_t s = 0; s < S; ++s) {
            for (int32_t h = 0; h < Hq && !lse_only; ++h) {
                float* o = out + s * o_ss + int64_t(t) * o_st + int64_t(h) * o_sh;
                for (int32_t d = lane; d < Dv; d += nlanes) o[d] = 0.0f;
            }
            for (int32_t h = lane; h < Hq; h += nlanes) lse[s * l_ss + int64_t(t) * l_st + h] = neg_inf();
        }
    }
}

// Tokens [tok0 + max_row_tokens, tok1) of a row whose real token count exceeds the host bound max_row_tokens are not
// attended (launches are sized by the bound): they are written as padding, (0, -inf) (their lse only with lse_only),
// in one partial (out and lse already offset to it).
__device__ __forceinline__ void fill_excess_tokens(float* out, int64_t o_st, int64_t o_sh, float* lse, int64_t l_st,
                                                   int32_t tok0, int32_t tok1, int32_t max_row_tokens, int32_t Hq,
                                                   int32_t Dv, int lane, int nlanes, bool lse_only) {
    const int32_t t_begin = tok0 + max(max_row_tokens, 0);
    if (t_begin < tok1) fill_padding(out, 0, o_st, o_sh, lse, 0, l_st, 1, Hq, Dv, t_begin, tok1, lane, nlanes, lse_only);
}

// The plans' per-(row, stripe) inputs: for every pair bs = b S + s of a workgroup's share, f(bs, ntok, lr) with ntok =
// row b's query tokens that are attended (at most max_row_tokens) and lr = the length of stripe stripe_begin + s of
// its context (clamped to [0, ctx_cap]). A thread takes four pairs at a time and issues their loads before using any,
// so a workgroup gathers 4 blockDim.x pairs in the time of one load.
template <class F>
__device__ __forceinline__ void for_each_plan_pair(const int32_t* row_start, const int32_t* ctx_len, int32_t B,
                                                   int32_t S, int32_t T, int32_t max_row_tokens, int32_t ctx_cap,
                                                   int32_t stripe_begin, int32_t P, int32_t I, F&& f) {
    const int32_t n = B * S;
    for (int32_t bs0 = threadIdx.x; bs0 < n; bs0 += 4 * blockDim.x) {
        int32_t q0[4], q1[4], cl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int32_t b = min(bs0 + u * int32_t(blockDim.x), n - 1) / S;
            q0[u] = row_start[b];
            q1[u] = row_start[b + 1];
            cl[u] = ctx_len[b];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int32_t bs = bs0 + u * int32_t(blockDim.x);
            if (bs >= n) break;
            const int32_t tok0 = min(max(q0[u], 0), T);
            const int32_t tok1 = min(max(q1[u], tok0), T);
            f(bs, min(tok1 - tok0, max_row_tokens),
              stripe_length(min(max(cl[u], 0), ctx_cap), stripe_begin + bs % S, P, I));
        }
    }
}

// Plans of the unit kernels: order[rank] = i for the n items whose keys (work estimates) sit in LDS, rank = the number
// of items with a larger key, or an equal key and a smaller index (longest first, ties in index order); an item whose
// key is negative (no work at all) is entered as -1, so its workgroup returns without looking at anything else. s_key holds
// rank_padded(n) entries, those past n set to -1 (below every real key). A workgroup of 256 threads ranks kRankItems
// items: kRankThreads threads share an item, each comparing it with its part of the keys, four at a time, and the
// parts' counts are summed through s_part (256 entries). Many small workgroups spread the n^2 comparisons over the
// whole chip.
constexpr int kRankThreads = 16;
constexpr int kRankItems = 256 / kRankThreads;
__host__ __device__ __forceinline__ int32_t rank_padded(int32_t n) {
    return (n + 4 * kRankThreads - 1) & ~(4 * kRankThreads - 1);
}

__device__ __forceinline__ void rank_longest_first(const int32_t* s_key, int32_t* s_part, int32_t n, int32_t* order) {
    const int32_t tid = threadIdx.x;
    const int32_t u = int32_t(blockIdx.x) * kRankItems + tid % kRankItems;
    const int32_t part = tid / kRankItems;
    int32_t rank = 0;
    if (u < n) {
        const int32_t mine = s_key[u];
        const int4* key4 = reinterpret_cast<const int4*>(s_key);
        const int32_t per = rank_padded(n) / (4 * kRankThreads);   // int4 entries of a part
#pragma unroll 4
        for (int32_t v4 = part * per; v4 < (part + 1) * per; ++v4) {
            const int4 o = key4[v4];
            const int32_t v = 4 * v4;
            rank += (o.x > mine) || (o.x == mine && v < u);
            rank += (o.y > mine) || (o.y == mine && v + 1 < u);
            rank += (o.z > mine) || (o.z == mine && v + 2 < u);
            rank += (o.w > mine) || (o.w == mine && v + 3 < u);
        }
    }
    s_part[tid] = rank;
    __syncthreads();
    if (tid < kRankItems && u < n) {
        int32_t r = 0;
#pragma unroll
        for (int k = 0; k < kRankThreads; ++k) r += s_part[k * kRankItems + tid];
        order[r] = s_key[u] < 0 ? -1 : u;
    }
}

}  // namespace cpattn
