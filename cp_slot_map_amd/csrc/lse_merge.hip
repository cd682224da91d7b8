// cp_lse_merge: exact combination of N attention partials by their log-sum-exps.
//
// The partials of a partitioned key set recombine exactly (mstar PR #1124, "Context / Sequence Parallel 1/5", PR
// description; dcp_combine and merge_attn_states in the vLLM compare view "[Core] Add explicit layer parallel plans",
// FlashAttentionImpl._forward_with_dcp): with M = max_i lse_i, lse = M + log sum_i exp(lse_i - M) and
// out = sum_i exp(lse_i - lse) * o_i. Empty partials (lse = -inf) weigh zero and are selected out, so their rows never
// reach the result.
//
// HBM-bound: one thread per (token, head, 4 dims) reads N float4 and N lse values (the lse loads hit cache across the
// Dv/4 threads of a (token, head)) and writes one float4 (or 4 bf16).
#include "common.h"

#include <cstdlib>

namespace cpattn {

struct MergeParams {
    const float* out_i[CPATTN_MAX_PARTIALS];
    const float* lse_i[CPATTN_MAX_PARTIALS];
    int64_t o_st[CPATTN_MAX_PARTIALS], o_sh[CPATTN_MAX_PARTIALS];
    int64_t l_st[CPATTN_MAX_PARTIALS], l_sh[CPATTN_MAX_PARTIALS];
    void* out;
    int64_t out_st, out_sh;
    float* lse_out;
    int64_t lse_out_st;
    const int32_t* token_count;
    int32_t N, T, H, Dv4;
};

// A thread handles 4 kV dims of a (token, head): kV float4 loads per partial in flight. NMAX >= N bounds the partial
// arrays (registers), so that wide threads stay within the register file when there are few partials.
template <bool kBf16Out, int kV, int NMAX>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeParams p) {
    const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int32_t Dq = p.Dv4 / kV;                        // threads per (token, head)
    const int64_t total = int64_t(p.T) * p.H * Dq;
    if (gid >= total) return;
    const int32_t d4 = int32_t(gid % Dq) * kV;            // first float4 of this thread
    const int64_t th = gid / Dq;
    const int32_t h = int32_t(th % p.H);
    const int32_t t = int32_t(th / p.H);

    // All loads are issued before any is used (one memory round trip). A partial whose lse is -inf is selected out,
    // never multiplied, so whatever its out row holds cannot reach the result.
    const bool padding = p.token_count != nullptr && t >= *p.token_count;
    float l[NMAX];
    f32x4_t o[NMAX][kV];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        if (i < p.N && !padding) {
            l[i] = p.lse_i[i][int64_t(t) * p.l_st[i] + int64_t(h) * p.l_sh[i]];
            const float* src = p.out_i[i] + int64_t(t) * p.o_st[i] + int64_t(h) * p.o_sh[i] + 4 * d4;
#pragma unroll
            for (int v = 0; v < kV; ++v) o[i][v] = *reinterpret_cast<const f32x4_t*>(src + 4 * v);
        } else {
            l[i] = neg_inf();
#pragma unroll
            for (int v = 0; v < kV; ++v) o[i][v] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        }
    }
    f32x4_t acc[kV];
    const float lse = lse_merge_rows<NMAX, kV>(l, o, acc);
    const int64_t off = int64_t(t) * p.out_st + int64_t(h) * p.out_sh + 4 * d4;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
        if (kBf16Out) {
            u32x2_t b = {pack2_bf16(acc[v][0], acc[v][1]), pack2_bf16(acc[v][2], acc[v][3])};
            *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.out) + off + 4 * v) = b;
        } else {
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + off + 4 * v) = acc[v];
        }
    }
    if (d4 == 0 && p.lse_out) p.lse_out[int64_t(t) * p.lse_out_st + h] = lse;
}

}  // namespace cpattn

using namespace cpattn;

extern "C" int32_t cp_lse_merge(const cp_merge_args* a, hipStream_t stream) {
    if (!a) return fail(CPATTN_EINVAL, "cp_lse_merge: args is null");
    if (a->num_partials < 1 || a->num_partials > CPATTN_MAX_PARTIALS)
        return fail(CPATTN_EINVAL, "num_partials = %d outside [1, %d]", a->num_partials, CPATTN_MAX_PARTIALS);
    if (a->num_tokens < 0 || a->num_heads < 0 || a->head_dim_v < 0)
        return fail(CPATTN_EINVAL, "negative size (T=%d, H=%d, Dv=%d)", a->num_tokens, a->num_heads, a->head_dim_v);
    if (a->head_dim_v % 4) return fail(CPATTN_EINVAL, "head_dim_v = %d must be a multiple of 4", a->head_dim_v);
    if (a->out_dtype != CPATTN_F32 && a->out_dtype != CPATTN_BF16)
        return fail(CPATTN_EINVAL, "out_dtype = %d unknown", a->out_dtype);
    const int64_t total = int64_t(a->num_tokens) * a->num_heads * (a->head_dim_v / 4);
    if (total == 0) return CPATTN_OK;
    if (!a->out) return fail(CPATTN_EINVAL, "cp_lse_merge: out is null");
    MergeParams p{};
    for (int i = 0; i < a->num_partials; ++i) {
        if (!a->part_out[i] || !a->part_lse[i]) return fail(CPATTN_EINVAL, "partial %d has a null pointer", i);
        if (static_cast<const void*>(a->part_out[i]) == a->out)
            return fail(CPATTN_EINVAL, "out aliases partial %d", i);
        if ((a->part_out_stride_token[i] % 4) || (a->part_out_stride_head[i] % 4) ||
            (reinterpret_cast<uintptr_t>(a->part_out[i]) % 16))
            return fail(CPATTN_EINVAL, "partial %d out must be 16-byte aligned with strides that are multiples of 4", i);
        p.out_i[i] = a->part_out[i];
        p.lse_i[i] = a->part_lse[i];
        p.o_st[i] = a->part_out_stride_token[i];
        p.o_sh[i] = a->part_out_stride_head[i];
        p.l_st[i] = a->part_lse_stride_token[i];
        p.l_sh[i] = a->part_lse_stride_head[i];
    }
    const int align = a->out_dtype == CPATTN_F32 ? 16 : 8;
    if ((reinterpret_cast<uintptr_t>(a->out) % align) || (a->out_stride_token % 4) || (a->out_stride_head % 4))
        return fail(CPATTN_EINVAL, "out must be %d-byte aligned with strides that are multiples of 4", align);
    p.out = a->out;
    p.out_st = a->out_stride_token;
    p.out_sh = a->out_stride_head;
    p.lse_out = a->lse_out;
    p.lse_out_st = a->lse_out_stride_token;
    p.token_count = a->token_count;
    p.N = a->num_partials;
    p.T = a->num_tokens;
    p.H = a->num_heads;
    p.Dv4 = a->head_dim_v / 4;
    // Dims a thread: 4 * kV with kV as large as Dv and the partial count allow (more bytes in flight per thread); the
    // partial arrays are sized for 5, 9 or 17 partials. Every output element is the same function of its inputs
    // whichever width serves it.
    const int nmax = a->num_partials <= 5 ? 5 : a->num_partials <= 9 ? 9 : 17;
    int kv = 1;
    if (nmax == 5 && a->head_dim_v % 16 == 0) kv = 4;
    else if (nmax <= 9 && a->head_dim_v % 8 == 0) kv = 2;
    const dim3 grid(uint32_t((total / kv + 255) / 256));
    const bool bf = a->out_dtype == CPATTN_BF16;
#define CPATTN_MERGE_LAUNCH(BF, KV, NM) hipLaunchKernelGGL((lse_merge_kernel<BF, KV, NM>), grid, dim3(256), 0, stream, p)
    if (nmax == 5) {
        if (kv == 4) { if (bf) CPATTN_MERGE_LAUNCH(true, 4, 5); else CPATTN_MERGE_LAUNCH(false, 4, 5); }
        else if (kv == 2) { if (bf) CPATTN_MERGE_LAUNCH(true, 2, 5); else CPATTN_MERGE_LAUNCH(false, 2, 5); }
        else { if (bf) CPATTN_MERGE_LAUNCH(true, 1, 5); else CPATTN_MERGE_LAUNCH(false, 1, 5); }
    } else if (nmax == 9) {
        if (kv == 2) { if (bf) CPATTN_MERGE_LAUNCH(true, 2, 9); else CPATTN_MERGE_LAUNCH(false, 2, 9); }
        else { if (bf) CPATTN_MERGE_LAUNCH(true, 1, 9); else CPATTN_MERGE_LAUNCH(false, 1, 9); }
    } else {
        if (bf) CPATTN_MERGE_LAUNCH(true, 1, 17); else CPATTN_MERGE_LAUNCH(false, 1, 17);
    }
#undef CPATTN_MERGE_LAUNCH
    return check_launch("cp_lse_merge");
}
