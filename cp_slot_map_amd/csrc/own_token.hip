// Own-token attention: causal attention of each row's in-step queries over the row's in-step K/V.
//
// When a row brings more than one token in a step, those tokens attend one another using the K/V that the layer hands
// over, apart from the pool (mstar PR #1124, "Context / Sequence Parallel 1/5", PR description); the vLLM compare view
// "[Core] Add explicit layer parallel plans" (FlashAttentionImpl._forward_with_dcp) passes the query offsets as the
// key offsets of this call. Query i of a row sees the row's keys 0..i. Only keys inside the row are ever addressed, so
// padding tokens of the bucket (and the keys of padding rows) are never read; padding outputs are (0, -inf).
//
// One wave per (row, kv head, block of R query rows); lanes split the head dim; each key updates the online softmax of
// the rows that may see it.
#include "launch.h"

namespace cpattn {

struct OwnParams {
    const void* q;
    int64_t q_st, q_sh;
    const void* k;
    const void* v;
    int64_t kv_st, kv_sh;
    float* out;
    int64_t o_st, o_sh;
    float* lse;
    int64_t l_st;
    const int32_t* cu;
    int32_t B, T, Hq, Hkv, G, max_row_tokens;
    float scale_log2;
    int32_t lse_only;   // CPATTN_FLAG_PAD_LSE_ONLY
};

template <typename T, int ND, int R>
__global__ __launch_bounds__(64) void own_token_generic_kernel(const OwnParams p) {
    const int lane = threadIdx.x;
    const int rb = blockIdx.x;
    const int b = blockIdx.y / p.Hkv;
    const int g = blockIdx.y % p.Hkv;
    const int32_t tok0 = min(max(p.cu[b], 0), p.T);
    const int32_t tok1 = min(max(p.cu[b + 1], tok0), p.T);
    if (g == 0 && rb == int(gridDim.x) - 1)
        fill_excess_tokens(p.out, p.o_st, p.o_sh, p.lse, p.l_st, tok0, tok1, p.max_row_tokens, p.Hq, ND * 64, lane, 64,
                           p.lse_only);
    const int32_t n = min(tok1 - tok0, p.max_row_tokens);
    const int32_t nrows = n * p.G;
    if (rb * R >= nrows) return;

    const T* Q = static_cast<const T*>(p.q);
    const T* K = static_cast<const T*>(p.k);
    const T* V = static_cast<const T*>(p.v);
    float q[R][ND];
    int32_t qi[R], head[R];
    bool valid[R];
    int32_t imax = 0;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int32_t rho = rb * R + rr;
        valid[rr] = rho < nrows;
        qi[rr] = valid[rr] ? rho / p.G : -1;
        head[rr] = g * p.G + (valid[rr] ? rho % p.G : 0);
        imax = max(imax, qi[rr]);
        const T* qp = Q + int64_t(tok0 + max(qi[rr], 0)) * p.q_st + int64_t(head[rr]) * p.q_sh;
#pragma unroll
        for (int i = 0; i < ND; ++i) q[rr][i] = valid[rr] ? load_f32(qp + lane + 64 * i) * p.scale_log2 : 0.f;
    }
    float m[R], l[R], acc[R][ND];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        m[rr] = neg_inf();
        l[rr] = 0.f;
#pragma unroll
        for (int i = 0; i < ND; ++i) acc[rr][i] = 0.f;
    }
    for (int32_t j = 0; j <= imax; ++j) {
        const int64_t off = int64_t(tok0 + j) * p.kv_st + int64_t(g) * p.kv_sh;
        float k[ND], v[ND];
#pragma unroll
        for (int i = 0; i < ND; ++i) {
            k[i] = load_f32(K + off + lane + 64 * i);
            v[i] = load_f32(V + off + lane + 64 * i);
        }
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            if (j > qi[rr]) continue;        // causal: wave-uniform condition (invalid rows have qi = -1)
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < ND; ++i) d = fmaf(q[rr][i], k[i], d);
            const float sc = wave_sum(d);
            const float mn = fmaxf(m[rr], sc);
            const float alpha = exp2f(m[rr] - mn);
            const float pj = exp2f(sc - mn);
            l[rr] = l[rr] * alpha + pj;
#pragma unroll
            for (int i = 0; i < ND; ++i) acc[rr][i] = fmaf(acc[rr][i], alpha, pj * v[i]);
            m[rr] = mn;
        }
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        if (!valid[rr]) continue;
        const int32_t t = tok0 + qi[rr];
        float* o = p.out + int64_t(t) * p.o_st + int64_t(head[rr]) * p.o_sh;
        const float inv = l[rr] > 0.f ? 1.0f / l[rr] : 0.f;
#pragma unroll
        for (int i = 0; i < ND; ++i) o[lane + 64 * i] = acc[rr][i] * inv;
        if (lane == 0)
            p.lse[int64_t(t) * p.l_st + head[rr]] = l[rr] > 0.f ? (m[rr] + log2f(l[rr])) * kLn2 : neg_inf();
    }
}

int32_t launch_own_token_generic(const cp_own_args& a, hipStream_t stream) {
    OwnParams p{};
    p.q = a.q;
    p.q_st = a.q_stride_token;
    p.q_sh = a.q_stride_head;
    p.k = a.k;
    p.v = a.v;
    p.kv_st = a.kv_stride_token;
    p.kv_sh = a.kv_stride_head;
    p.out = a.out;
    p.o_st = a.out_stride_token;
    p.o_sh = a.out_stride_head;
    p.lse = a.lse;
    p.l_st = a.lse_stride_token;
    p.cu = a.cu_seqlens;
    p.B = a.num_rows;
    p.T = a.bucket_tokens;
    p.Hq = a.num_q_heads;
    p.Hkv = a.num_kv_heads;
    p.G = a.num_q_heads / a.num_kv_heads;
    p.max_row_tokens = a.max_row_tokens;
    p.scale_log2 = a.scale * kLog2e;
    p.lse_only = (a.flags & CPATTN_FLAG_PAD_LSE_ONLY) ? 1 : 0;
    if (int32_t st = launch_pad(a.out, 0, a.out_stride_token, a.out_stride_head, a.lse, 0, a.lse_stride_token,
                                a.cu_seqlens, a.num_rows, a.bucket_tokens, 1, a.num_q_heads, a.head_dim,
                                (a.flags & CPATTN_FLAG_PAD_LSE_ONLY) != 0, stream))
        return st;
    if (a.num_rows == 0) return CPATTN_OK;
    constexpr int R = 8;
    // (at least one block of query rows: it also writes tokens past an understated max_row_tokens as padding)
    const int64_t rows = int64_t(std::max(1, a.max_row_tokens)) * p.G;
    const dim3 grid(uint32_t((rows + R - 1) / R), uint32_t(a.num_rows * a.num_kv_heads));
    const bool f32 = a.dtype == CPATTN_F32;
    if (a.head_dim == 64) {
        if (f32)
            hipLaunchKernelGGL((own_token_generic_kernel<float, 1, R>), grid, dim3(64), 0, stream, p);
        else
            hipLaunchKernelGGL((own_token_generic_kernel<uint16_t, 1, R>), grid, dim3(64), 0, stream, p);
    } else {
        if (f32)
            hipLaunchKernelGGL((own_token_generic_kernel<float, 2, R>), grid, dim3(64), 0, stream, p);
        else
            hipLaunchKernelGGL((own_token_generic_kernel<uint16_t, 2, R>), grid, dim3(64), 0, stream, p);
    }
    return check_launch("cp_own_token_attn");
}

}  // namespace cpattn
