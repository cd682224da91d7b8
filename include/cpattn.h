/*
 * cpattn: attention over a context-parallel striped paged KV pool, for AMD Instinct MI355X (gfx950).
 *
 * The method (mstar PR #1124, "Context / Sequence Parallel 1/5: split the KV cache by position across GPUs (DCP)",
 * PR description and commit message): a paged pool with context parallelism spreads each page's token slots over P
 * partners. The token in logical slot s is kept by partner s mod P at index floor(s / P) of that partner's pool, and
 * page ids stay logical. Each partner attends the slots it holds and returns a partial output together with that
 * partial's log-sum-exp; the partials are combined without approximation. When a row brings several tokens in one
 * step, they also attend each other, using the K/V the layer hands over, and that partial joins the combination. The vLLM compare view
 * "[Core] Add explicit layer parallel plans" (FlashAttentionImpl._forward_with_dcp) shows the same shape: context
 * attention over the paged cache with (out, lse), a combine across ranks, own-token attention with the query offsets
 * used as key offsets, and a final LSE merge.
 *
 * On one GPU every stripe's pool is resident, so the exchange between partners is simply the merge reading the
 * partial buffers.
 *
 * Conventions for every entry point:
 *   - Every call returns a status: CPATTN_OK, CPATTN_EINVAL (an argument is wrong), CPATTN_EUNSUPPORTED (valid but no
 *     kernel is built for it, e.g. a head dim) or CPATTN_ELAUNCH (the HIP launch failed). On any non-OK status
 *     nothing was enqueued; cpattn_last_error() gives a message for the calling thread. Nothing asserts or throws.
 *   - All validation that can be done on the host happens before anything is enqueued. Values that live in device
 *     memory (lengths, block tables, offsets) cannot be checked there; kernels clamp them so that no access leaves
 *     the buffers described by the arguments (see each entry point).
 *   - Tensor arguments are device pointers owned by the caller. The library allocates no device memory and keeps no
 *     pointer after the call returns, apart from the work it queued on `stream`. Calls are asynchronous on `stream`
 *     (NULL = the null stream).
 *   - Strides are in elements. The innermost (head-dim) axis of every tensor is contiguous.
 *   - LSEs are natural-log log-sum-exps of the scaled scores, fp32. An empty key set gives out = 0 and lse = -inf.
 */
#ifndef CPATTN_H_
#define CPATTN_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPATTN_OK 0
#define CPATTN_EINVAL 1
#define CPATTN_EUNSUPPORTED 2
#define CPATTN_ELAUNCH 3

#define CPATTN_F32 0
#define CPATTN_BF16 1
#define CPATTN_FP8_E4M3 2   /* element type of fp8 pools and rows (cp_kv_write, cp_debug_gather_stripe): OCP 8-bit
                               E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities) */

/* cp_paged_args.kv_format: what the pools hold. The vLLM compare view "[Core] Add explicit layer parallel plans" passes
 * per-tensor k_descale / v_descale to its attention calls; a key or value element stands for its code's value times
 * the tensor's descale. */
#define CPATTN_KV_SAME 0       /* pools have the element type of q (dtype) */
#define CPATTN_KV_FP8_E4M3 1   /* pools hold CPATTN_FP8_E4M3 codes, dequantized with k_descale / v_descale */

#define CPATTN_GQA 0
#define CPATTN_MLA 1

/* P <= 16 stripes plus the own-token partial. */
#define CPATTN_MAX_PARTIALS 17

/* cp_paged_args.flags */
#define CPATTN_FLAG_FIXED_SPLITS 1   /* see cp_paged_attn_partial: results independent of the rest of the call */
#define CPATTN_FLAG_PAD_LSE_ONLY 2   /* padding tokens get lse = -inf only; their out rows are not written (cp_lse_merge
                                        selects a -inf partial out and never reads its row, and with token_count it
                                        reads no padding token at all) */

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* cpattn_last_error(void);

/* Library version string, e.g. "0.1.0". */
const char* cpattn_version(void);

/* sizeof() of the argument structs, for bindings to check their layout: which = 0 cp_paged_args, 1 cp_own_args,
 * 2 cp_merge_args, 3 cp_merge_out. Returns -1 for an unknown `which`. */
int64_t cpattn_struct_size(int32_t which);

/*
 * cp_slot_map: logical slot -> (partner, physical slot); the write-addressing path.
 *
 * Source: the slot rule of mstar PR #1124 (PR description); the review thread on resident planning notes that a
 * partner pool holds page_size / P slots a page, which is why every write path must go through this map.
 *
 * Interleave: the vLLM compare view "[Core] Add explicit layer parallel plans" reads a KV-cache interleave size I
 * from the parallel config (FlashAttentionMetadataBuilder); the pages give no placement for it, and the one taken
 * here is that runs of I consecutive slots go to one partner, partners in turn, each partner packing its runs:
 * partner floor(s / I) mod P at physical slot floor(s / (I P)) * I + s mod I. I = 1 is the PR's rule.
 *
 *   logical_slot  device int64 [n]: page_id * page_size + offset of each token to write; < 0 marks a padding token.
 *   interleave    I >= 1; I * P must divide page_size.
 *   partner_out   device int32 [n]: floor(s / I) mod P (s mod P for I = 1), or -1 for s < 0.
 *   phys_out      device int64 [n]: floor(s / (I P)) * I + s mod I (floor(s / P) for I = 1; always
 *                 page_id * (page_size / P) + a slot below page_size / P), or -1 for s < 0.
 * EINVAL: n < 0, P < 1, I < 1, page_size < 1, page_size % (I * P) != 0, or a null pointer with n > 0. n = 0 enqueues
 * nothing.
 */
int32_t cp_slot_map(const int64_t* logical_slot, int64_t n, int32_t page_size, int32_t num_partners,
                    int32_t interleave, int32_t* partner_out, int64_t* phys_out, hipStream_t stream);

/*
 * cp_slot_map_rank: the per-rank write view. Rank `rank` writes a token it owns at its physical slot and every other
 * token at `sink_slot` (a slot of the sink page in its own pool), as the PR description states for non-owners.
 *   write_slot_out  device int64 [n]: physical slot for owned tokens, sink_slot otherwise, -1 for s < 0.
 * EINVAL: as cp_slot_map, plus rank outside [0, P) or sink_slot < 0.
 */
int32_t cp_slot_map_rank(const int64_t* logical_slot, int64_t n, int32_t page_size, int32_t num_partners,
                         int32_t interleave, int32_t rank, int64_t sink_slot, int64_t* write_slot_out,
                         hipStream_t stream);

/*
 * cp_kv_write: fused slot map + write of K (and V) rows into the stripe pools, for stripes
 * [stripe_begin, stripe_begin + stripe_count) held by the caller.
 *
 * Source: every write-addressing path must go through the placement, and a token is written by its owner and to the
 * sink page on every other rank (mstar PR #1124, PR description and commit message; the review thread on resident
 * planning shows what goes wrong when a write path skips it).
 *
 *   logical_slot  device int64 [n]; < 0 = padding (written nowhere).
 *   dtype         CPATTN_F32, CPATTN_BF16 or CPATTN_FP8_E4M3 (codes copied as bytes): element type of rows and pools.
 *   k_src         device [n, num_kv_heads, head_dim] (token stride src_stride_token, head stride src_stride_head).
 *   v_src         device [n, num_kv_heads, head_dim_v] with the same strides, or NULL (MLA: the latent row is K).
 *   pools         layout of cp_paged_args (element (r, page, slot, g, d) at pool + r*kv_stride_stripe + ...).
 *   interleave    I >= 1: the placement of cp_slot_map (I = 1: partner s mod P at floor(s / P)).
 *   sink_slot     >= 0: stripes in range that do not own a token write it to this physical slot (per-rank view);
 *                 < 0: only the owner writes (all stripes resident on one device).
 * A token whose page id falls outside [0, num_pages) is not written. Tokens sharing a destination race (last wins).
 * EINVAL: bad geometry (as cp_slot_map), stripe range, null pointers, negative sizes or strides,
 * sink_slot >= num_pages * page_size / P.
 */
int32_t cp_kv_write(const int64_t* logical_slot, int64_t n, const void* k_src, const void* v_src,
                    int64_t src_stride_token, int64_t src_stride_head, int32_t dtype, int32_t num_kv_heads,
                    int32_t head_dim, int32_t head_dim_v, void* k_pool, void* v_pool, int64_t kv_stride_stripe,
                    int64_t kv_stride_page, int64_t kv_stride_slot, int64_t kv_stride_head, int32_t page_size,
                    int32_t num_partners, int32_t interleave, int32_t num_pages, int32_t stripe_begin,
                    int32_t stripe_count, int64_t sink_slot, hipStream_t stream);

/*
 * Arguments of cp_paged_attn_partial.
 *
 * Query layout: q element (token t, head h, dim d) at q + t*q_stride_token + h*q_stride_head + d, tokens of row b
 * being [q_row_start[b], q_row_start[b+1]). Tokens in [q_row_start[num_rows], num_tokens) are padding.
 *
 * Pool layout: element (stripe r, page p, slot j, kv head g, dim d) of the K pool is at
 *   k_pool + r*kv_stride_stripe + p*kv_stride_page + j*kv_stride_slot + g*kv_stride_head + d,
 * the same for v_pool. Stripe r's pool has num_pages pages of page_size / P slots; page ids are the logical ones
 * from the block table. For MLA each slot holds one latent row of head_dim (576) values: the key is the whole row and
 * the value its first head_dim_v (512) columns; v_pool must equal k_pool and kv_stride_head is ignored.
 *
 * Partial layout (S = stripe_count, stripe index relative to stripe_begin):
 *   out (s, t, h, d) at out + s*out_stride_stripe + t*out_stride_token + h*out_stride_head + d   (fp32)
 *   lse (s, t, h)    at lse + s*lse_stride_stripe + t*lse_stride_token + h                     (fp32)
 */
typedef struct cp_paged_args {
    int32_t kind;             /* CPATTN_GQA or CPATTN_MLA */
    int32_t dtype;            /* element type of q, k_pool, v_pool: CPATTN_F32 or CPATTN_BF16 */
    int32_t num_rows;         /* B: rows (requests) */
    int32_t num_tokens;       /* T: query tokens in the (possibly padded) bucket */
    int32_t num_partners;     /* P: stripes of the pool; must divide page_size */
    int32_t stripe_begin;     /* first stripe attended by this call */
    int32_t stripe_count;     /* S: stripes attended; out and lse hold S partials */
    int32_t page_size;        /* logical page size (slots of a logical page) */
    int32_t num_pages;        /* pages in each stripe pool; block-table entries outside [0, num_pages) read page 0 */
    int32_t num_q_heads;      /* Hq */
    int32_t num_kv_heads;     /* Hkv; Hq % Hkv == 0; query head h reads kv head h / (Hq / Hkv) */
    int32_t head_dim;         /* qk dim: 64 or 128 (GQA), 576 (MLA) */
    int32_t head_dim_v;       /* value dim: equal to head_dim (GQA), 512 (MLA) */
    float scale;              /* softmax scale applied to q.k */
    int32_t max_ctx_len;      /* host upper bound of ctx_len[b]; sizes the launch and the workspace. A row whose device
                                 ctx_len exceeds it is taken as its first max_ctx_len tokens (every kernel clamps) */
    int32_t max_row_tokens;   /* host upper bound of a row's query tokens, sizes the launch; a row's tokens past it are
                                 not attended and come out as padding (0, -inf) */
    int32_t max_pages;        /* block-table entries used per row; ctx_len[b] is clamped to max_pages * page_size */
    int32_t flags;            /* CPATTN_FLAG_FIXED_SPLITS | CPATTN_FLAG_PAD_LSE_ONLY; other bits are EINVAL */
    int32_t interleave;       /* KV-cache interleave size I (0 or 1: none); the placement of cp_slot_map; I * P must
                                 divide page_size */
    int32_t kv_format;        /* CPATTN_KV_SAME or CPATTN_KV_FP8_E4M3 (dtype bf16 only) */
    float k_descale;          /* fp8 pools: a key element is its code's value times k_descale (finite, > 0) */
    float v_descale;          /* fp8 pools: a value element is its code's value times v_descale (finite, > 0);
                                 MLA: equal to k_descale (one latent tensor) */
    const int32_t* q_row_start;  /* device int32 [num_rows + 1], non-decreasing, q_row_start[num_rows] <= num_tokens */
    const int32_t* ctx_len;      /* device int32 [num_rows]: context tokens of row b in the pool (all stripes) */
    const int32_t* block_table;  /* device int32 [num_rows, bt_stride]: logical page ids */
    int64_t bt_stride;
    const void* q;
    int64_t q_stride_token, q_stride_head;
    const void* k_pool;
    const void* v_pool;
    int64_t kv_stride_stripe, kv_stride_page, kv_stride_slot, kv_stride_head;
    float* out;
    int64_t out_stride_stripe, out_stride_token, out_stride_head;
    float* lse;
    int64_t lse_stride_stripe, lse_stride_token;
    void* workspace;          /* device scratch of cp_paged_attn_workspace_size() bytes (NULL if that is 0); no
                                 initial contents are required and it holds nothing useful after the call. Calls
                                 that share a workspace must be ordered (e.g. on one stream). */
    int64_t workspace_bytes;
} cp_paged_args;

/*
 * cp_paged_attn_partial: per-stripe paged attention returning out + lse, for every stripe r in
 * [stripe_begin, stripe_begin + stripe_count).
 *
 * Source: each partner attends the slots it holds and returns its partial with the partial's log-sum-exp (mstar
 * PR #1124, PR description; the PR also notes that a decode kernel without an LSE output cannot be used because the
 * merge needs it); context attention over the paged cache through the block table returning (out, lse) in the vLLM
 * compare view, FlashAttentionImpl._forward_with_dcp.
 *
 * For every real query token t of row b, head h and stripe r: the keys are the context positions p < ctx_len[b] with
 * floor(p / I) mod P == r (p mod P == r without interleave: the slots partner r holds); local token i of stripe r is
 * position floor(i / I) * I * P + r * I + i mod I (i*P + r for I = 1), found at page block_table[b][i / (page_size/P)],
 * slot i % (page_size/P) of r's pool, for every I. Every query token of a row sees the whole
 * context (no mask). Rows with ctx_len[b] <= r give (0, -inf). Padding tokens get out = 0 and lse = -inf (with
 * CPATTN_FLAG_PAD_LSE_ONLY lse = -inf only, their out rows untouched) and their queries are not read.
 *
 * Rounding. A stripe's keys may be split into pieces that are merged exactly; only the rounding of the result depends
 * on where the splits fall. By default the bf16 head_dim-128 decode path balances the whole call's work over the
 * device's resident waves, so split points, and the last bits of a row's result, depend on the rest of the call (other
 * rows, the stripe range) and on the device's compute-unit count; identical calls on one device give identical bits.
 * With CPATTN_FLAG_FIXED_SPLITS the splits fall at fixed key offsets of each stripe, so a row's result is the same to
 * the bit whatever else the call holds (e.g. one stripe alone equals that stripe of an all-stripes call), at some cost
 * in speed when context lengths vary widely.
 *
 * fp8 pools (kv_format CPATTN_KV_FP8_E4M3): every element read from the pools is decoded exactly and multiplied by
 * its descale in fp32 (the key descale folded into the score scale, the value descale applied to the normalised
 * output).
 *
 * Precision. Scores and sums accumulate in fp32. The value product weights by the probabilities held to about 16
 * significant bits (bf16 GQA calls with at most 16 query rows, Hq / Hkv per token, per row and kv head: a bf16 pair
 * high + residual) or 11 (bf16 GQA calls with more query rows, and bf16 MLA: fp16 weights, with the values widened to
 * fp16 for that product, so bf16 value elements must stay below 65504 in magnitude; every E4M3 code fits), and every
 * output is normalised by the sum of the weights actually applied.
 *
 * EINVAL: a null args/pointer, unknown flag bits, interleave < 0, an unknown kv_format, fp8 pools with dtype other
 * than bf16, a descale that is not finite and positive or MLA with k_descale != v_descale, Hq % Hkv != 0, page_size % (I * P) != 0, a stripe range outside [0, P), negative sizes or
 * strides, bt_stride < max_pages, too small a workspace, MLA with Hkv != 1 or v_pool != k_pool.
 * EUNSUPPORTED: a (kind, dtype, head_dim, head_dim_v) with no kernel. Built: GQA f32/bf16 with (64, 64) and
 * (128, 128), bf16 queries over fp8 pools for both; MLA bf16 with (576, 512), also over fp8 latent pools.
 */
int32_t cp_paged_attn_partial(const cp_paged_args* args, hipStream_t stream);

/* Workspace bytes cp_paged_attn_partial needs for `args` (depends on shapes and the host bounds only; the pointers in
 * `args` are not looked at). EINVAL/EUNSUPPORTED as cp_paged_attn_partial for everything but pointers. */
int32_t cp_paged_attn_workspace_size(const cp_paged_args* args, int64_t* bytes_out);

/*
 * Merged output of cp_paged_attn_merged.
 *   out (t, h, d) at out + t*out_stride_token + h*out_stride_head + d, fp32 or bf16 (round to nearest even);
 *   lse (t, h) at lse + t*lse_stride_token + h (fp32, natural log; nullable).
 */
typedef struct cp_merge_out {
    int32_t out_dtype;        /* CPATTN_F32 or CPATTN_BF16 */
    int32_t reserved0;
    void* out;
    int64_t out_stride_token, out_stride_head;
    float* lse;
    int64_t lse_stride_token;
} cp_merge_out;

/*
 * cp_paged_attn_merged: every stripe's partial and their exact merge, in one call, when all P stripes are resident on
 * the device (stripe_begin = 0, stripe_count = P).
 *
 * Source: each partner's partial with its log-sum-exp, then the exact merge of the partials (mstar PR #1124, PR
 * description); on one device the exchange between partners is the merge reading resident partials, so the step can
 * finish the split pieces of each stripe and merge the stripes in the same pass.
 *
 * Results: exactly those of cp_paged_attn_partial(args) followed by cp_lse_merge of its S partials with token_count =
 * q_row_start + num_rows (the same bits): args->out / args->lse receive the per-stripe partials and `merged` the merged
 * output; tokens at or past q_row_start[num_rows] come out as (0, -inf). On the bf16 head_dim-128 decode path with the
 * default schedule the fix-up of split pieces and the merge run as one kernel after the partial kernel; every other
 * path runs the partial call and the merge call back to back.
 * EINVAL: as cp_paged_attn_partial; a null `merged` or merged->out (num_tokens > 0); stripe_begin != 0 or
 * stripe_count != P; an unknown out_dtype; merged->out not 16-byte aligned or strides not multiples of 8 elements;
 * merged->out equal to args->out.
 */
int32_t cp_paged_attn_merged(const cp_paged_args* args, const cp_merge_out* merged, hipStream_t stream);

/*
 * cp_paged_attn_partial_noalloc: cp_paged_attn_partial for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same entry point, kernels and results,
 * with the workspace taken from a static device array of cp_paged_attn_noalloc_scratch_bytes() bytes (64 MiB) that
 * the library holds on every device it runs on until the process ends, instead of args->workspace (ignored).
 *
 * Nothing is allocated, by the library or any library it calls; the caller still passes q, the pools and the out/lse
 * buffers. The scratch needs no initial contents. Every call on one device shares that device's scratch: calls that
 * overlap on one device (different streams without ordering between them) race and give undefined results; calls
 * ordered on one stream are safe.
 * EINVAL: as cp_paged_attn_partial, and a call whose workspace would exceed the static scratch (see
 * cp_paged_attn_workspace_size; the bf16 decode schedule needs about 4-17 MB on MI355X, the bf16 extend kernel's
 * unit order at most 32 KB, MLA up to a few hundred MB for small batches whose stripes are split into many chunks).
 * ELAUNCH: the scratch address could not be obtained.
 */
int32_t cp_paged_attn_partial_noalloc(const cp_paged_args* args, hipStream_t stream);

/* Size in bytes of the static scratch of cp_paged_attn_partial_noalloc (per device). */
int64_t cp_paged_attn_noalloc_scratch_bytes(void);

/*
 * Arguments of cp_own_token_attn.
 *   q (t, h, d) at q + t*q_stride_token + h*q_stride_head + d; k and v (t, g, d) at k/v + t*kv_stride_token +
 *   g*kv_stride_head + d; out (t, h, d) at out + t*out_stride_token + h*out_stride_head + d; lse (t, h) at
 *   lse + t*lse_stride_token + h.
 */
typedef struct cp_own_args {
    int32_t dtype;            /* CPATTN_F32 or CPATTN_BF16, for q, k, v */
    int32_t num_rows;         /* real rows; row b owns bucket tokens [cu_seqlens[b], cu_seqlens[b+1]) */
    int32_t bucket_tokens;    /* tokens in the bucket; [cu_seqlens[num_rows], bucket_tokens) is padding */
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;         /* 64 or 128 */
    float scale;
    int32_t max_row_tokens;   /* host upper bound of a row's tokens (sizes the launch); a row's tokens past it are not
                                 attended and come out as padding (0, -inf) */
    int32_t flags;            /* 0 or CPATTN_FLAG_PAD_LSE_ONLY; other bits are EINVAL */
    int32_t reserved0;
    const int32_t* cu_seqlens;   /* device int32 [num_rows + 1], non-decreasing; values are clamped to the bucket */
    const void* q;
    int64_t q_stride_token, q_stride_head;
    const void* k;
    const void* v;
    int64_t kv_stride_token, kv_stride_head;
    float* out;
    int64_t out_stride_token, out_stride_head;
    float* lse;
    int64_t lse_stride_token;
} cp_own_args;

/*
 * cp_own_token_attn: causal attention of each row's in-step queries over the row's in-step K/V.
 *
 * Source: when a row brings more than one token in a step, those tokens also attend one another, using the K/V that
 * the layer hands over rather than the pool, and in a padded (captured) bucket the keys of padding rows must stay
 * invisible to this kernel (mstar PR #1124, PR description; its review thread on the padding test reports NaN in
 * padding keys spreading to every real row when padding rows sat in the bucket); the own-token call in the vLLM
 * compare view passes the query offsets as the key offsets.
 *
 * Query i of a row (0-based within the row) sees the row's keys 0..i. Keys and queries of padding tokens are never
 * read; padding tokens get out = 0 and lse = -inf (with CPATTN_FLAG_PAD_LSE_ONLY lse = -inf only, their out rows
 * untouched). Precision: fp32 scores and sums; bf16 calls at head_dim 128 weight the values by fp16-rounded
 * probabilities with the values widened to fp16 (bf16 values must stay below 65504 in magnitude), normalised by the
 * sum of those weights; other calls compute in fp32.
 * EINVAL: null pointers, negative sizes, Hq % Hkv != 0, unknown flag bits. EUNSUPPORTED: head_dim other than 64 or
 * 128.
 */
int32_t cp_own_token_attn(const cp_own_args* args, hipStream_t stream);

/*
 * Arguments of cp_lse_merge. Partial i: out (t, h, d) at part_out[i] + t*part_out_stride_token[i] +
 * h*part_out_stride_head[i] + d and lse (t, h) at part_lse[i] + t*part_lse_stride_token[i] + h*part_lse_stride_head[i].
 * Output (t, h, d) at out + t*out_stride_token + h*out_stride_head + d; lse_out (t, h) at lse_out +
 * t*lse_out_stride_token + h.
 */
typedef struct cp_merge_args {
    int32_t num_partials;     /* N in [1, CPATTN_MAX_PARTIALS] */
    int32_t num_tokens;       /* T */
    int32_t num_heads;        /* H */
    int32_t head_dim_v;       /* Dv, a multiple of 4 */
    int32_t out_dtype;        /* CPATTN_F32 or CPATTN_BF16 (round to nearest even) */
    int32_t reserved0;
    const int32_t* token_count;  /* nullable device int32 [1]: tokens >= *token_count are padding: written as
                                    (0, -inf) without reading the partials */
    const float* part_out[CPATTN_MAX_PARTIALS];
    const float* part_lse[CPATTN_MAX_PARTIALS];
    int64_t part_out_stride_token[CPATTN_MAX_PARTIALS];
    int64_t part_out_stride_head[CPATTN_MAX_PARTIALS];
    int64_t part_lse_stride_token[CPATTN_MAX_PARTIALS];
    int64_t part_lse_stride_head[CPATTN_MAX_PARTIALS];
    void* out;
    int64_t out_stride_token, out_stride_head;
    float* lse_out;           /* nullable */
    int64_t lse_out_stride_token;
} cp_merge_args;

/*
 * cp_lse_merge: exact combination of N partials by their LSEs.
 *
 * Source: the partials are merged exactly (mstar PR #1124, PR description); dcp_combine and merge_attn_states in the
 * vLLM compare view, FlashAttentionImpl._forward_with_dcp.
 *
 * M = max_i lse_i; M = -inf gives out = 0, lse = -inf; otherwise lse = M + log sum_i exp(lse_i - M) and
 * out = sum_i exp(lse_i - lse) * o_i. A partial with lse_i = -inf contributes nothing: it is selected out, never
 * multiplied, so its out row may hold anything (NaN included). Tokens >= *token_count are not read at all.
 * EINVAL: N outside [1, CPATTN_MAX_PARTIALS], null pointers, Dv % 4 != 0, negative sizes, out aliasing a partial.
 */
int32_t cp_lse_merge(const cp_merge_args* args, hipStream_t stream);

/*
 * cp_stripe_length: how many of a row's context tokens stripe r holds (host call; nothing is enqueued).
 *
 * Source: the slot rule of mstar PR #1124 (PR description) places logical slot s on partner s mod P; with P dividing
 * page_size the row's context position t lands on partner t mod P, so stripe r holds the positions r, r + P, ... below
 * ctx_len: ceil((ctx_len - r) / P) of them (0 when ctx_len <= r). With an interleave size I (the placement of
 * cp_slot_map) it holds the positions t with floor(t / I) mod P == r. This is the stripe length every attention kernel
 * uses (the same function), exported so that callers and tests size per-stripe buffers from the library's own rule.
 *   len_out  host int32: the stripe length.
 * EINVAL: P outside [1, 16], I < 1, page_size % (I * P) != 0, r outside [0, P), ctx_len < 0, len_out null.
 */
int32_t cp_stripe_length(int32_t ctx_len, int32_t page_size, int32_t num_partners, int32_t interleave, int32_t r,
                         int32_t* len_out);

/*
 * cp_debug_gather_stripe (test support): copy stripe r's keys of one row, in local order, into a dense buffer, through
 * the same device addressing function the attention kernels use, so page addressing can be checked bit for bit.
 *   dst (i, g, d) at dst + (i*num_kv_heads + g)*head_dim + d for i below stripe r's length (cp_stripe_length), same
 *   dtype as the pool; dst_rows is its capacity in rows (tokens).
 *   rows_out: host int32, set to the number of rows written (the stripe length) when the call is accepted.
 *   block_table_row: device int32 [>= ceil(ctx_len / page_size)].
 * EINVAL: bad geometry, r outside [0, P), null pointers, negative sizes, dst_rows below the stripe length.
 */
int32_t cp_debug_gather_stripe(const void* k_pool, int32_t dtype, int64_t kv_stride_stripe, int64_t kv_stride_page,
                               int64_t kv_stride_slot, int64_t kv_stride_head, int32_t num_pages,
                               const int32_t* block_table_row, int32_t ctx_len, int32_t page_size,
                               int32_t num_partners, int32_t interleave, int32_t r, int32_t num_kv_heads,
                               int32_t head_dim, void* dst, int64_t dst_rows, int32_t* rows_out, hipStream_t stream);

/*
 * cp_debug_stream_read (measurement support): read `bytes` bytes at `src` (device, 16-byte aligned, bytes a multiple
 * of 16) once, sequentially, with coalesced 16-byte loads, and write one 32-bit XOR of what each workgroup read into
 * sink[0 .. blocks) (device, caller-owned, sink_words >= 1 words; blocks = min(sink_words, what the size needs)). Its
 * duration gives the read bandwidth a plain stream reaches on the device, the achievable denominator next to the
 * nominal HBM peak when the attention kernels' KV rate is reported. Asynchronous on `stream`.
 * EINVAL: negative size, bytes not a multiple of 16, src misaligned, sink_words < 1, null pointers (bytes > 0).
 */
int32_t cp_debug_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t sink_words, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H_ */
