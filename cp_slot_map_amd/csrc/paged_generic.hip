// Generic per-stripe paged attention partial (out + natural-log lse), any built dtype and head dims.
//
// Each partner attends only the slots it holds and returns its partial with the partial's log-sum-exp (mstar PR #1124,
// "Context / Sequence Parallel 1/5", PR description); the vLLM compare view "[Core] Add explicit layer parallel plans"
// (FlashAttentionImpl._forward_with_dcp) runs this context attention over the paged cache through the block table.
//
// One wave per (row, stripe, kv head, block of R query rows). Lanes split the head dim; for each of the stripe's keys
// the wave reduces R dot products, and every lane keeps an online softmax state (running max in log2 units, running
// sum, weighted value accumulator) for its R rows. This path favours clarity over speed; the bf16 GQA decode shape has
// its own MFMA kernel.
#include "launch.h"

namespace cpattn {

struct GenericParams {
    const void* q;
    int64_t q_st, q_sh;
    const void* kp;
    const void* vp;
    PoolGeom geo;
    const int32_t* q_row_start;
    const int32_t* ctx_len;
    const int32_t* bt;
    int64_t bt_stride;
    float* out;
    int64_t o_ss, o_st, o_sh;
    float* lse;
    int64_t l_ss, l_st;
    int32_t B, T, P, stripe_begin, Hq, Hkv, G, max_pages, page_size, max_row_tokens;
    int32_t ctx_cap;        // context lengths are clamped to min(max_pages * page_size, max_ctx_len)
    float scale_log2;   // softmax scale (times the key descale for fp8 pools) in log2 units
    float v_scale;      // value descale of fp8 pools, else 1
    int32_t lse_only;   // CPATTN_FLAG_PAD_LSE_ONLY
};

// T: element type of q; TKV: element type of the pools (T itself, or uint8_t for fp8 codes).
template <typename T, typename TKV, int NQ, int NV, int R>
__global__ __launch_bounds__(64) void paged_generic_kernel(const GenericParams p) {
    const int lane = threadIdx.x;
    const int rb = blockIdx.x;
    const int b = blockIdx.y / p.Hkv;
    const int g = blockIdx.y % p.Hkv;
    const int s = blockIdx.z;

    int32_t tok0 = min(max(p.q_row_start[b], 0), p.T);
    int32_t tok1 = min(max(p.q_row_start[b + 1], tok0), p.T);
    if (g == 0 && rb == int(gridDim.x) - 1)
        fill_excess_tokens(p.out + s * p.o_ss, p.o_st, p.o_sh, p.lse + s * p.l_ss, p.l_st, tok0, tok1, p.max_row_tokens,
                           p.Hq, NV * 64, lane, 64, p.lse_only);
    const int32_t ntok = min(tok1 - tok0, p.max_row_tokens);
    const int32_t nrows = ntok * p.G;
    if (rb * R >= nrows) return;

    const int32_t r = p.stripe_begin + s;
    const int32_t L = min(max(p.ctx_len[b], 0), p.ctx_cap);
    const int32_t Lr = stripe_length(L, r, p.P, p.geo.interleave);
    const int32_t* bt_row = p.bt + int64_t(b) * p.bt_stride;
    const T* Q = static_cast<const T*>(p.q);
    const TKV* K = static_cast<const TKV*>(p.kp);
    const TKV* V = static_cast<const TKV*>(p.vp);

    float q[R][NQ];
    int32_t tok[R], head[R];
    bool valid[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int32_t rho = rb * R + rr;
        valid[rr] = rho < nrows;
        tok[rr] = tok0 + (valid[rr] ? rho / p.G : 0);
        head[rr] = g * p.G + (valid[rr] ? rho % p.G : 0);
        const T* qp = Q + int64_t(tok[rr]) * p.q_st + int64_t(head[rr]) * p.q_sh;
#pragma unroll
        for (int i = 0; i < NQ; ++i) q[rr][i] = valid[rr] ? load_f32(qp + lane + 64 * i) * p.scale_log2 : 0.f;
    }

    float m[R], l[R], acc[R][NV];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        m[rr] = neg_inf();
        l[rr] = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[rr][i] = 0.f;
    }

    for (int32_t j = 0; j < Lr; ++j) {
        const int64_t off = stripe_token_offset(bt_row, j, r, g, p.geo);
        float k[NQ], v[NV];
#pragma unroll
        for (int i = 0; i < NQ; ++i) k[i] = load_f32(K + off + lane + 64 * i);
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = load_f32(V + off + lane + 64 * i);
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < NQ; ++i) d = fmaf(q[rr][i], k[i], d);
            const float sc = wave_sum(d);
            const float mn = fmaxf(m[rr], sc);
            const float alpha = exp2f(m[rr] - mn);
            const float pj = exp2f(sc - mn);
            l[rr] = l[rr] * alpha + pj;
#pragma unroll
            for (int i = 0; i < NV; ++i) acc[rr][i] = fmaf(acc[rr][i], alpha, pj * v[i]);
            m[rr] = mn;
        }
    }

#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        if (!valid[rr]) continue;
        float* o = p.out + s * p.o_ss + int64_t(tok[rr]) * p.o_st + int64_t(head[rr]) * p.o_sh;
        const float inv = l[rr] > 0.f ? 1.0f / l[rr] : 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) o[lane + 64 * i] = acc[rr][i] * inv * p.v_scale;
        if (lane == 0)
            p.lse[s * p.l_ss + int64_t(tok[rr]) * p.l_st + head[rr]] =
                l[rr] > 0.f ? (m[rr] + log2f(l[rr])) * kLn2 : neg_inf();
    }
}

struct PadParams {
    float* out;
    int64_t o_ss, o_st, o_sh;
    float* lse;
    int64_t l_ss, l_st;
    const int32_t* q_row_start;
    int32_t B, T, S, Hq, Dv, tokens_per_block;
    int32_t lse_only;    // CPATTN_FLAG_PAD_LSE_ONLY
};

__global__ __launch_bounds__(64) void pad_partials_kernel(const PadParams p) {
    const int32_t first = min(max(p.q_row_start[p.B], 0), p.T);
    const int32_t t0 = max(int32_t(blockIdx.x) * p.tokens_per_block, first);
    const int32_t t1 = min(int32_t(blockIdx.x + 1) * p.tokens_per_block, p.T);
    if (t0 >= t1) return;
    fill_padding(p.out, p.o_ss, p.o_st, p.o_sh, p.lse, p.l_ss, p.l_st, p.S, p.Hq, p.Dv, t0, t1, threadIdx.x, 64,
                 p.lse_only);
}

int32_t launch_pad(float* out, int64_t o_ss, int64_t o_st, int64_t o_sh, float* lse, int64_t l_ss, int64_t l_st,
                   const int32_t* starts, int32_t B, int32_t T, int32_t S, int32_t Hq, int32_t Dv, bool lse_only,
                   hipStream_t stream) {
    if (T == 0) return CPATTN_OK;
    PadParams p{out, o_ss, o_st, o_sh, lse, l_ss, l_st, starts, B, T, S, Hq, Dv, 4, lse_only ? 1 : 0};
    const dim3 grid(uint32_t((T + 3) / 4));
    hipLaunchKernelGGL(pad_partials_kernel, grid, dim3(64), 0, stream, p);
    return check_launch("padding fill");
}

int32_t launch_pad_partials(const cp_paged_args& a, hipStream_t stream) {
    return launch_pad(a.out, a.out_stride_stripe, a.out_stride_token, a.out_stride_head, a.lse, a.lse_stride_stripe,
                      a.lse_stride_token, a.q_row_start, a.num_rows, a.num_tokens, a.stripe_count, a.num_q_heads,
                      a.head_dim_v, (a.flags & CPATTN_FLAG_PAD_LSE_ONLY) != 0, stream);
}

template <typename T, typename TKV, int NQ, int NV, int R>
static void launch_generic_t(const GenericParams& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((paged_generic_kernel<T, TKV, NQ, NV, R>), grid, dim3(64), 0, stream, p);
}

int32_t launch_paged_generic(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream) {
    GenericParams p{};
    p.q = a.q;
    p.q_st = a.q_stride_token;
    p.q_sh = a.q_stride_head;
    p.kp = a.k_pool;
    p.vp = a.v_pool;
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
    p.Hq = a.num_q_heads;
    p.Hkv = a.num_kv_heads;
    p.G = a.num_q_heads / a.num_kv_heads;
    p.max_pages = a.max_pages;
    p.ctx_cap = ctx_cap_of(a);
    p.page_size = a.page_size;
    p.max_row_tokens = a.max_row_tokens;
    const bool fp8 = a.kv_format == CPATTN_KV_FP8_E4M3;
    p.scale_log2 = a.scale * (fp8 ? a.k_descale : 1.0f) * kLog2e;
    p.v_scale = fp8 ? a.v_descale : 1.0f;
    p.lse_only = (a.flags & CPATTN_FLAG_PAD_LSE_ONLY) ? 1 : 0;

    if (int32_t st = launch_pad_partials(a, stream)) return st;
    if (a.num_rows == 0) return CPATTN_OK;
    // (at least one block of query rows: it also writes tokens past an understated max_row_tokens as padding)
    const int64_t rows = int64_t(std::max(1, a.max_row_tokens)) * p.G;
    const bool f32 = a.dtype == CPATTN_F32;
    if (a.kind == CPATTN_MLA) {
        constexpr int R = 8;
        dim3 grid(uint32_t((rows + R - 1) / R), uint32_t(a.num_rows), uint32_t(a.stripe_count));
        if (fp8)
            launch_generic_t<uint16_t, uint8_t, 9, 8, R>(p, grid, stream);
        else
            launch_generic_t<uint16_t, uint16_t, 9, 8, R>(p, grid, stream);
    } else if (a.head_dim == 64) {
        constexpr int R = 8;
        dim3 grid(uint32_t((rows + R - 1) / R), uint32_t(a.num_rows * a.num_kv_heads), uint32_t(a.stripe_count));
        if (f32)
            launch_generic_t<float, float, 1, 1, R>(p, grid, stream);
        else if (fp8)
            launch_generic_t<uint16_t, uint8_t, 1, 1, R>(p, grid, stream);
        else
            launch_generic_t<uint16_t, uint16_t, 1, 1, R>(p, grid, stream);
    } else {
        constexpr int R = 8;
        dim3 grid(uint32_t((rows + R - 1) / R), uint32_t(a.num_rows * a.num_kv_heads), uint32_t(a.stripe_count));
        if (f32)
            launch_generic_t<float, float, 2, 2, R>(p, grid, stream);
        else if (fp8)
            launch_generic_t<uint16_t, uint8_t, 2, 2, R>(p, grid, stream);
        else
            launch_generic_t<uint16_t, uint16_t, 2, 2, R>(p, grid, stream);
    }
    return check_launch("cp_paged_attn_partial (generic)");
}

// --------------------------------------------------------------------------------- debug gather of one stripe
template <typename T>
__global__ void gather_stripe_kernel(const T* __restrict__ pool, PoolGeom geo, const int32_t* __restrict__ bt_row,
                                     int32_t Lr, int32_t r, int32_t Hkv, int32_t D, T* __restrict__ dst) {
    const int64_t total = int64_t(Lr) * Hkv * D;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
         e += int64_t(gridDim.x) * blockDim.x) {
        const int32_t d = int32_t(e % D);
        const int64_t ig = e / D;
        const int32_t g = int32_t(ig % Hkv);
        const int32_t i = int32_t(ig / Hkv);
        dst[e] = pool[stripe_token_offset(bt_row, i, r, g, geo) + d];
    }
}

}  // namespace cpattn

using namespace cpattn;

extern "C" int32_t cp_stripe_length(int32_t ctx_len, int32_t page_size, int32_t num_partners, int32_t interleave,
                                    int32_t r, int32_t* len_out) {
    if (num_partners < 1 || num_partners > 16 || interleave < 1 || page_size < 1 || page_size % num_partners ||
        (page_size / num_partners) % interleave)
        return fail(CPATTN_EINVAL, "bad geometry (page_size=%d, P=%d, interleave=%d)", page_size, num_partners,
                    interleave);
    if (r < 0 || r >= num_partners) return fail(CPATTN_EINVAL, "stripe %d outside [0, %d)", r, num_partners);
    if (ctx_len < 0) return fail(CPATTN_EINVAL, "ctx_len = %d is negative", ctx_len);
    if (!len_out) return fail(CPATTN_EINVAL, "cp_stripe_length: len_out is null");
    *len_out = stripe_length(ctx_len, r, num_partners, interleave);
    return CPATTN_OK;
}

extern "C" int32_t cp_debug_gather_stripe(const void* k_pool, int32_t dtype, int64_t kv_stride_stripe,
                                          int64_t kv_stride_page, int64_t kv_stride_slot, int64_t kv_stride_head,
                                          int32_t num_pages, const int32_t* block_table_row, int32_t ctx_len,
                                          int32_t page_size, int32_t num_partners, int32_t interleave, int32_t r,
                                          int32_t num_kv_heads, int32_t head_dim, void* dst, int64_t dst_rows,
                                          int32_t* rows_out, hipStream_t stream) {
    int32_t Lr = 0;
    if (int32_t st = cp_stripe_length(ctx_len, page_size, num_partners, interleave, r, &Lr)) return st;
    if (num_kv_heads < 1 || head_dim < 1 || num_pages < 1) return fail(CPATTN_EINVAL, "negative or zero size");
    if (kv_stride_stripe < 0 || kv_stride_page < 0 || kv_stride_slot < 0 || kv_stride_head < 0)
        return fail(CPATTN_EINVAL, "negative stride");
    if (dtype != CPATTN_F32 && dtype != CPATTN_BF16 && dtype != CPATTN_FP8_E4M3)
        return fail(CPATTN_EINVAL, "dtype %d unknown", dtype);
    if (!rows_out) return fail(CPATTN_EINVAL, "cp_debug_gather_stripe: rows_out is null");
    if (dst_rows < Lr)
        return fail(CPATTN_EINVAL, "cp_debug_gather_stripe: stripe %d holds %d tokens, dst has room for %lld", r, Lr,
                    (long long)dst_rows);
    *rows_out = Lr;
    if (Lr == 0) return CPATTN_OK;
    if (!k_pool || !block_table_row || !dst) return fail(CPATTN_EINVAL, "cp_debug_gather_stripe: null pointer");
    PoolGeom geo{kv_stride_stripe, kv_stride_page, kv_stride_slot, kv_stride_head, page_size / num_partners,
                 ilog2_exact(page_size / num_partners), num_pages, interleave};
    const int64_t total = int64_t(Lr) * num_kv_heads * head_dim;
    const dim3 grid(uint32_t(std::min<int64_t>((total + 255) / 256, 65536)));
    if (dtype == CPATTN_F32)
        hipLaunchKernelGGL(gather_stripe_kernel<float>, grid, dim3(256), 0, stream,
                           static_cast<const float*>(k_pool), geo, block_table_row, Lr, r, num_kv_heads, head_dim,
                           static_cast<float*>(dst));
    else if (dtype == CPATTN_FP8_E4M3)
        hipLaunchKernelGGL(gather_stripe_kernel<uint8_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint8_t*>(k_pool), geo, block_table_row, Lr, r, num_kv_heads, head_dim,
                           static_cast<uint8_t*>(dst));
    else
        hipLaunchKernelGGL(gather_stripe_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(k_pool), geo, block_table_row, Lr, r, num_kv_heads, head_dim,
                           static_cast<uint16_t*>(dst));
    return check_launch("cp_debug_gather_stripe");
}
