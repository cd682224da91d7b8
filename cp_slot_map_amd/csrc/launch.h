// Internal launch interface between the validating entry points and the kernel files.
#pragma once

#include "common.h"

namespace cpattn {

// Interleave size of a call (0 in the struct means 1) and the longest stripe of a row with max_ctx_len tokens (stripe
// 0 holds the most); host-side bounds size launches and workspaces from it.
inline int32_t interleave_of(const cp_paged_args& a) { return a.interleave > 1 ? a.interleave : 1; }
// The context length every kernel uses for row b: ctx_len[b] clamped to [0, ctx_cap], ctx_cap the smaller of what the
// block table can address and the host's bound max_ctx_len (launch sizes and workspaces follow max_ctx_len, so a
// larger device value must not reach them).
inline int32_t ctx_cap_of(const cp_paged_args& a) {
    const int64_t cap = std::min<int64_t>(int64_t(a.max_pages) * a.page_size, a.max_ctx_len > 0 ? a.max_ctx_len : 0);
    return int32_t(cap);
}

inline int64_t max_stripe_length(const cp_paged_args& a) {
    return stripe_length(a.max_ctx_len > 0 ? a.max_ctx_len : 0, 0, a.num_partners, interleave_of(a));
}

// Generic per-stripe partial: any built (dtype, head_dim, head_dim_v), any pp. One wave per (row, stripe, kv head,
// block of query rows) streams the whole stripe; used for fp32 pools, MLA until its own kernel takes over, and any
// shape the specialised kernels do not cover.
int32_t launch_paged_generic(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream);

// Specialised bf16 GQA partial (head_dim = head_dim_v = 128) with MFMA score and value products and split chunks.
bool decode_bf16_eligible(const cp_paged_args& a, const PoolGeom& geo);
int64_t decode_bf16_workspace_bytes(const cp_paged_args& a);
int64_t decode_bf16_workspace_bytes_on_device(const cp_paged_args& a, const PoolGeom& geo);
// With m non-null (and decode_bf16_fuses_merge), the stripes' partials are also merged into m in the same launches.
bool decode_bf16_fuses_merge(const cp_paged_args& a);
int32_t launch_paged_decode_bf16(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream,
                                 const cp_merge_out* m = nullptr);

// Specialised bf16 GQA partial for rows that bring many query tokens (head_dim = head_dim_v = 128): 128 query rows per
// workgroup, K/V tiles staged in LDS, MFMA score and value products. The same kernel serves the own-token part.
bool extend_bf16_eligible(const cp_paged_args& a, const PoolGeom& geo);
int32_t launch_paged_extend_bf16(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream);
int64_t extend_bf16_workspace_bytes(const cp_paged_args& a);
bool own_bf16_eligible(const cp_own_args& a);
int32_t launch_own_token_bf16(const cp_own_args& a, hipStream_t stream);

// Specialised bf16 MLA partial (one latent head of 576, values its first 512; 16, 32, 64 or 128 query heads) with MFMA
// score and value products over latent tiles staged in LDS.
bool mla_decode_eligible(const cp_paged_args& a, const PoolGeom& geo);
int64_t mla_decode_workspace_bytes(const cp_paged_args& a);
int32_t launch_mla_decode(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream);

// (0, -inf) for the padding tokens [q_row_start[num_rows], num_tokens) of all S partials.
int32_t launch_pad_partials(const cp_paged_args& a, hipStream_t stream);

// (0, -inf) for tokens [starts[B], T) of S outputs with Hq heads of Dv values (starts is a device array).
int32_t launch_pad(float* out, int64_t o_ss, int64_t o_st, int64_t o_sh, float* lse, int64_t l_ss, int64_t l_st,
                   const int32_t* starts, int32_t B, int32_t T, int32_t S, int32_t Hq, int32_t Dv, bool lse_only,
                   hipStream_t stream);

// Own-token causal attention (generic: f32/bf16, head_dim 64 or 128).
int32_t launch_own_token_generic(const cp_own_args& a, hipStream_t stream);

}  // namespace cpattn
