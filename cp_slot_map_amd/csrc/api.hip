// Entry points of libcpattn: host-side validation and kernel dispatch. Nothing is enqueued unless every check that
// can be made on the host passes; device-resident values are clamped inside the kernels.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "launch.h"

// Scratch of cp_paged_attn_partial_noalloc: a file-scope device array, one copy on every device the library runs on,
// held until the process ends. Host code never uses its name as an address: the address of the current device's copy
// comes from hipGetSymbolAddress, once per device, and that pointer is what the kernels receive.
#define CPATTN_NOALLOC_SCRATCH_BYTES (int64_t(64) << 20)
static __device__ __align__(256) unsigned char scratch[CPATTN_NOALLOC_SCRATCH_BYTES];

namespace cpattn {

static thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int32_t check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CPATTN_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
    return CPATTN_OK;
}

static bool negative_stride(const cp_paged_args& a) {
    return a.q_stride_token < 0 || a.q_stride_head < 0 || a.kv_stride_stripe < 0 || a.kv_stride_page < 0 ||
           a.kv_stride_slot < 0 || a.kv_stride_head < 0 || a.out_stride_stripe < 0 || a.out_stride_token < 0 ||
           a.out_stride_head < 0 || a.lse_stride_stripe < 0 || a.lse_stride_token < 0 || a.bt_stride < 0;
}

// Validate cp_paged_args; on success fill the pool geometry.
static int32_t check_paged(const cp_paged_args* pa, PoolGeom* geo) {
    if (!pa) return fail(CPATTN_EINVAL, "cp_paged_attn_partial: args is null");
    const cp_paged_args& a = *pa;
    if (a.kind != CPATTN_GQA && a.kind != CPATTN_MLA) return fail(CPATTN_EINVAL, "kind = %d unknown", a.kind);
    if (a.dtype != CPATTN_F32 && a.dtype != CPATTN_BF16) return fail(CPATTN_EINVAL, "dtype = %d unknown", a.dtype);
    if (a.flags & ~(CPATTN_FLAG_FIXED_SPLITS | CPATTN_FLAG_PAD_LSE_ONLY))
        return fail(CPATTN_EINVAL, "flags = %#x has unknown bits", a.flags);
    if (a.num_rows < 0 || a.num_tokens < 0 || a.max_ctx_len < 0 || a.max_row_tokens < 0 || a.max_pages < 0)
        return fail(CPATTN_EINVAL, "negative size");
    if (a.num_partners < 1 || a.num_partners > 16)
        return fail(CPATTN_EINVAL, "num_partners = %d outside [1, 16]", a.num_partners);
    if (a.kv_format != CPATTN_KV_SAME && a.kv_format != CPATTN_KV_FP8_E4M3)
        return fail(CPATTN_EINVAL, "kv_format = %d unknown", a.kv_format);
    if (a.kv_format == CPATTN_KV_FP8_E4M3) {
        if (a.dtype != CPATTN_BF16) return fail(CPATTN_EINVAL, "fp8 pools are read with bf16 queries (dtype = %d)", a.dtype);
        if (!(a.k_descale > 0.f && a.k_descale < INFINITY) || !(a.v_descale > 0.f && a.v_descale < INFINITY))
            return fail(CPATTN_EINVAL, "fp8 descales must be finite and positive (k %g, v %g)", double(a.k_descale),
                        double(a.v_descale));
        // MLA keys and values are the same latent rows, so they carry one descale.
        if (a.kind == CPATTN_MLA && a.k_descale != a.v_descale)
            return fail(CPATTN_EINVAL, "MLA latent rows have one descale (k %g != v %g)", double(a.k_descale),
                        double(a.v_descale));
    }
    if (a.interleave < 0 || a.interleave > 65536) return fail(CPATTN_EINVAL, "interleave = %d outside [0, 65536]", a.interleave);
    const int32_t ilv = interleave_of(a);
    if (a.page_size < 1 || a.page_size % (a.num_partners * ilv))
        return fail(CPATTN_EINVAL, "num_partners * interleave = %d must divide page_size = %d", a.num_partners * ilv,
                    a.page_size);
    if (a.stripe_count < 1 || a.stripe_begin < 0 || a.stripe_begin + a.stripe_count > a.num_partners)
        return fail(CPATTN_EINVAL, "stripes [%d, %d) outside [0, %d)", a.stripe_begin, a.stripe_begin + a.stripe_count,
                    a.num_partners);
    if (a.num_pages < 1) return fail(CPATTN_EINVAL, "num_pages = %d must be >= 1 (page 0 is the sink)", a.num_pages);
    if (a.num_q_heads < 1 || a.num_kv_heads < 1 || a.num_q_heads % a.num_kv_heads)
        return fail(CPATTN_EINVAL, "num_q_heads = %d must be a positive multiple of num_kv_heads = %d", a.num_q_heads,
                    a.num_kv_heads);
    if (a.bt_stride < a.max_pages) return fail(CPATTN_EINVAL, "bt_stride < max_pages");
    if (negative_stride(a)) return fail(CPATTN_EINVAL, "negative stride");
    if (int64_t(a.max_pages) * a.page_size > (int64_t(1) << 31) - 1)
        return fail(CPATTN_EINVAL, "max_pages * page_size overflows int32");
    if (a.kind == CPATTN_MLA) {
        if (a.num_kv_heads != 1) return fail(CPATTN_EINVAL, "MLA needs num_kv_heads = 1 (one latent head)");
        if (a.v_pool != a.k_pool) return fail(CPATTN_EINVAL, "MLA reads values from the latent rows: v_pool != k_pool");
        if (a.dtype != CPATTN_BF16 || a.head_dim != 576 || a.head_dim_v != 512)
            return fail(CPATTN_EUNSUPPORTED, "MLA is built for bf16 with head_dim 576, head_dim_v 512");
    } else {
        if (a.head_dim != a.head_dim_v || (a.head_dim != 64 && a.head_dim != 128))
            return fail(CPATTN_EUNSUPPORTED, "GQA is built for head_dim = head_dim_v in {64, 128} (got %d, %d)",
                        a.head_dim, a.head_dim_v);
    }
    const int32_t pp = a.page_size / a.num_partners;
    *geo = PoolGeom{a.kv_stride_stripe, a.kv_stride_page, a.kv_stride_slot, a.kv_stride_head, pp, ilog2_exact(pp),
                    a.num_pages, ilv};
    return CPATTN_OK;
}

// Pointer checks of a call that launches (the workspace-size query takes the shapes only).
static int32_t check_paged_pointers(const cp_paged_args& a) {
    if (a.num_tokens > 0 && (!a.out || !a.lse)) return fail(CPATTN_EINVAL, "out/lse is null");
    if (a.num_rows > 0 && (!a.q_row_start || !a.ctx_len || !a.block_table || !a.q || !a.k_pool || !a.v_pool))
        return fail(CPATTN_EINVAL, "null device pointer");
    if (a.num_tokens > 0 && !a.q_row_start) return fail(CPATTN_EINVAL, "q_row_start is null");
    return CPATTN_OK;
}

static int64_t paged_workspace(const cp_paged_args& a, const PoolGeom& geo) {
    if (extend_bf16_eligible(a, geo)) return extend_bf16_workspace_bytes(a);
    if (decode_bf16_eligible(a, geo)) return decode_bf16_workspace_bytes(a);
    if (mla_decode_eligible(a, geo)) return mla_decode_workspace_bytes(a);
    return 0;
}

// Scratch bytes a call touches on the current device (at most paged_workspace()).
static int64_t paged_workspace_on_device(const cp_paged_args& a, const PoolGeom& geo) {
    if (extend_bf16_eligible(a, geo)) return extend_bf16_workspace_bytes(a);
    if (decode_bf16_eligible(a, geo)) return decode_bf16_workspace_bytes_on_device(a, geo);
    if (mla_decode_eligible(a, geo)) return mla_decode_workspace_bytes(a);
    return 0;
}

static int32_t dispatch_paged(const cp_paged_args& a, const PoolGeom& geo, hipStream_t stream) {
    if (a.num_tokens == 0) return CPATTN_OK;
    if (extend_bf16_eligible(a, geo)) return launch_paged_extend_bf16(a, geo, stream);
    if (decode_bf16_eligible(a, geo)) return launch_paged_decode_bf16(a, geo, stream);
    if (mla_decode_eligible(a, geo)) return launch_mla_decode(a, geo, stream);
    return launch_paged_generic(a, geo, stream);
}

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch` (looked up once per device, with that device current).
static int32_t device_scratch(void** out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CPATTN_ELAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(CPATTN_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t g = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (g != hipSuccess || !ptr)
            return fail(CPATTN_ELAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(g));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return CPATTN_OK;
}

}  // namespace cpattn

using namespace cpattn;

extern "C" const char* cpattn_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* cpattn_version(void) { return "0.1.0"; }

extern "C" int64_t cpattn_struct_size(int32_t which) {
    switch (which) {
        case 0: return int64_t(sizeof(cp_paged_args));
        case 1: return int64_t(sizeof(cp_own_args));
        case 2: return int64_t(sizeof(cp_merge_args));
        case 3: return int64_t(sizeof(cp_merge_out));
        default: return -1;
    }
}

extern "C" int32_t cp_paged_attn_workspace_size(const cp_paged_args* a, int64_t* bytes_out) {
    PoolGeom geo;
    if (int32_t st = check_paged(a, &geo)) return st;
    if (!bytes_out) return fail(CPATTN_EINVAL, "bytes_out is null");
    *bytes_out = paged_workspace(*a, geo);
    return CPATTN_OK;
}

extern "C" int32_t cp_paged_attn_partial(const cp_paged_args* a, hipStream_t stream) {
    PoolGeom geo;
    if (int32_t st = check_paged(a, &geo)) return st;
    if (int32_t st = check_paged_pointers(*a)) return st;
    const int64_t need = paged_workspace(*a, geo);
    if (need > 0 && (!a->workspace || a->workspace_bytes < need))
        return fail(CPATTN_EINVAL, "workspace of %lld bytes needed (got %lld)", (long long)need,
                    (long long)a->workspace_bytes);
    return dispatch_paged(*a, geo, stream);
}

extern "C" int32_t cp_paged_attn_merged(const cp_paged_args* a, const cp_merge_out* m, hipStream_t stream) {
    PoolGeom geo;
    if (int32_t st = check_paged(a, &geo)) return st;
    if (int32_t st = check_paged_pointers(*a)) return st;
    if (!m) return fail(CPATTN_EINVAL, "cp_paged_attn_merged: merged is null");
    if (a->stripe_begin != 0 || a->stripe_count != a->num_partners)
        return fail(CPATTN_EINVAL, "cp_paged_attn_merged merges all resident stripes: stripes [%d, %d) of %d",
                    a->stripe_begin, a->stripe_begin + a->stripe_count, a->num_partners);
    if (m->out_dtype != CPATTN_F32 && m->out_dtype != CPATTN_BF16)
        return fail(CPATTN_EINVAL, "merged out_dtype = %d unknown", m->out_dtype);
    if (a->num_tokens > 0 && !m->out) return fail(CPATTN_EINVAL, "merged out is null");
    if ((reinterpret_cast<uintptr_t>(m->out) & 15) || (m->out_stride_token & 7) || (m->out_stride_head & 7) ||
        m->out_stride_token < 0 || m->out_stride_head < 0 || m->lse_stride_token < 0)
        return fail(CPATTN_EINVAL, "merged out must be 16-byte aligned with non-negative strides that are multiples of 8");
    if (m->out == a->out) return fail(CPATTN_EINVAL, "merged out aliases the partials");
    const int64_t need = paged_workspace(*a, geo);
    if (need > 0 && (!a->workspace || a->workspace_bytes < need))
        return fail(CPATTN_EINVAL, "workspace of %lld bytes needed (got %lld)", (long long)need,
                    (long long)a->workspace_bytes);
    if (a->num_tokens == 0) return CPATTN_OK;
    if (decode_bf16_eligible(*a, geo) && !extend_bf16_eligible(*a, geo) && decode_bf16_fuses_merge(*a))
        return launch_paged_decode_bf16(*a, geo, stream, m);
    if (int32_t st = dispatch_paged(*a, geo, stream)) return st;
    cp_merge_args ma{};
    ma.num_partials = a->stripe_count;
    ma.num_tokens = a->num_tokens;
    ma.num_heads = a->num_q_heads;
    ma.head_dim_v = a->head_dim_v;
    ma.out_dtype = m->out_dtype;
    ma.token_count = a->q_row_start + a->num_rows;
    for (int32_t i = 0; i < a->stripe_count; ++i) {
        ma.part_out[i] = a->out + i * a->out_stride_stripe;
        ma.part_lse[i] = a->lse + i * a->lse_stride_stripe;
        ma.part_out_stride_token[i] = a->out_stride_token;
        ma.part_out_stride_head[i] = a->out_stride_head;
        ma.part_lse_stride_token[i] = a->lse_stride_token;
        ma.part_lse_stride_head[i] = 1;
    }
    ma.out = m->out;
    ma.out_stride_token = m->out_stride_token;
    ma.out_stride_head = m->out_stride_head;
    ma.lse_out = m->lse;
    ma.lse_out_stride_token = m->lse_stride_token;
    return cp_lse_merge(&ma, stream);
}

extern "C" int64_t cp_paged_attn_noalloc_scratch_bytes(void) { return CPATTN_NOALLOC_SCRATCH_BYTES; }

extern "C" int32_t cp_paged_attn_partial_noalloc(const cp_paged_args* a, hipStream_t stream) {
    PoolGeom geo;
    if (int32_t st = check_paged(a, &geo)) return st;
    if (int32_t st = check_paged_pointers(*a)) return st;
    const int64_t need = paged_workspace_on_device(*a, geo);
    if (need > CPATTN_NOALLOC_SCRATCH_BYTES)
        return fail(CPATTN_EINVAL, "cp_paged_attn_partial_noalloc: this call needs %lld bytes of scratch, the static "
                    "scratch holds %lld; use cp_paged_attn_partial with a workspace", (long long)need,
                    (long long)CPATTN_NOALLOC_SCRATCH_BYTES);
    cp_paged_args b = *a;
    b.workspace = nullptr;
    b.workspace_bytes = 0;
    if (need > 0) {
        void* ptr = nullptr;
        if (int32_t st = device_scratch(&ptr)) return st;
        b.workspace = ptr;
        b.workspace_bytes = CPATTN_NOALLOC_SCRATCH_BYTES;
    }
    return dispatch_paged(b, geo, stream);
}

extern "C" int32_t cp_own_token_attn(const cp_own_args* pa, hipStream_t stream) {
    if (!pa) return fail(CPATTN_EINVAL, "cp_own_token_attn: args is null");
    const cp_own_args& a = *pa;
    if (a.dtype != CPATTN_F32 && a.dtype != CPATTN_BF16) return fail(CPATTN_EINVAL, "dtype = %d unknown", a.dtype);
    if (a.num_rows < 0 || a.bucket_tokens < 0 || a.max_row_tokens < 0) return fail(CPATTN_EINVAL, "negative size");
    if (a.flags & ~CPATTN_FLAG_PAD_LSE_ONLY) return fail(CPATTN_EINVAL, "flags = %#x has unknown bits", a.flags);
    if (a.num_q_heads < 1 || a.num_kv_heads < 1 || a.num_q_heads % a.num_kv_heads)
        return fail(CPATTN_EINVAL, "num_q_heads = %d must be a positive multiple of num_kv_heads = %d", a.num_q_heads,
                    a.num_kv_heads);
    if (a.head_dim != 64 && a.head_dim != 128)
        return fail(CPATTN_EUNSUPPORTED, "own-token attention is built for head_dim 64 and 128 (got %d)", a.head_dim);
    if (a.q_stride_token < 0 || a.q_stride_head < 0 || a.kv_stride_token < 0 || a.kv_stride_head < 0 ||
        a.out_stride_token < 0 || a.out_stride_head < 0 || a.lse_stride_token < 0)
        return fail(CPATTN_EINVAL, "negative stride");
    if (a.bucket_tokens == 0) return CPATTN_OK;
    if (!a.cu_seqlens || !a.out || !a.lse) return fail(CPATTN_EINVAL, "null device pointer");
    if (a.num_rows > 0 && (!a.q || !a.k || !a.v)) return fail(CPATTN_EINVAL, "null device pointer");
    if (own_bf16_eligible(a)) return launch_own_token_bf16(a, stream);
    return launch_own_token_generic(a, stream);
}
