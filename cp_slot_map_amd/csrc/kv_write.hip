// cp_kv_write: the write path of a context-parallel pool, slot map fused with the copy into the stripe pools.
//
// Every write goes through the placement (mstar PR #1124, "Context / Sequence Parallel 1/5", PR description and commit
// message): logical slot s belongs to partner s mod P at physical slot floor(s / P), i.e. page floor(s / P) / pp and
// slot floor(s / P) mod pp of that partner's pool (pp = page_size / P); with interleave I, partner floor(s / I) mod P
// at physical slot floor(s / (I P)) * I + s mod I (the placement of cp_slot_map). Non-owners write the sink slot when
// one is given. The review thread on resident planning is the counter-example: addressing at the logical page size writes
// every token on every rank at offsets the smaller physical pages do not have.
//
// One 64-lane wave per (token, stripe in range): lanes copy the head rows with 16-byte (or narrower) accesses.
#include "common.h"

namespace cpattn {

struct KvWriteParams {
    const int64_t* slot;
    const uint8_t* k_src;
    const uint8_t* v_src;
    int64_t src_st, src_sh;          // bytes
    uint8_t* kp;
    uint8_t* vp;
    int64_t s_stripe, s_page, s_slot, s_head;   // bytes
    int64_t n;
    int64_t P, I, pp, num_pages, sink;
    int32_t stripe_begin, stripe_count, Hkv, row_k_bytes, row_v_bytes;
};

__device__ __forceinline__ void copy_row(uint8_t* dst, const uint8_t* src, int32_t bytes, int lane) {
    if ((bytes & 15) == 0 && ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15) == 0) {
        for (int32_t o = lane * 16; o < bytes; o += 64 * 16)
            *reinterpret_cast<u32x4_t*>(dst + o) = *reinterpret_cast<const u32x4_t*>(src + o);
    } else if ((bytes & 1) == 0 && ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 1) == 0) {
        for (int32_t o = lane * 2; o < bytes; o += 64 * 2)
            *reinterpret_cast<uint16_t*>(dst + o) = *reinterpret_cast<const uint16_t*>(src + o);
    } else {
        for (int32_t o = lane; o < bytes; o += 64) dst[o] = src[o];
    }
}

__global__ __launch_bounds__(64) void kv_write_kernel(const KvWriteParams p) {
    const int64_t w = blockIdx.x;
    const int64_t i = w / p.stripe_count;
    const int32_t r = p.stripe_begin + int32_t(w % p.stripe_count);
    if (i >= p.n) return;
    const int64_t s = p.slot[i];
    if (s < 0) return;
    int32_t owner;
    int64_t phys;
    place_slot(s, p.P, p.I, owner, phys);
    if (owner != r) {
        if (p.sink < 0) return;
        phys = p.sink;
    }
    const int64_t page = phys / p.pp;
    const int64_t sl = phys - page * p.pp;
    if (page >= p.num_pages) return;
    const int64_t base = int64_t(r) * p.s_stripe + page * p.s_page + sl * p.s_slot;
    const int lane = threadIdx.x;
    for (int32_t g = 0; g < p.Hkv; ++g) {
        copy_row(p.kp + base + g * p.s_head, p.k_src + i * p.src_st + g * p.src_sh, p.row_k_bytes, lane);
        if (p.v_src) copy_row(p.vp + base + g * p.s_head, p.v_src + i * p.src_st + g * p.src_sh, p.row_v_bytes, lane);
    }
}

}  // namespace cpattn

using namespace cpattn;

extern "C" int32_t cp_kv_write(const int64_t* logical_slot, int64_t n, const void* k_src, const void* v_src,
                               int64_t src_stride_token, int64_t src_stride_head, int32_t dtype, int32_t num_kv_heads,
                               int32_t head_dim, int32_t head_dim_v, void* k_pool, void* v_pool,
                               int64_t kv_stride_stripe, int64_t kv_stride_page, int64_t kv_stride_slot,
                               int64_t kv_stride_head, int32_t page_size, int32_t num_partners, int32_t interleave,
                               int32_t num_pages, int32_t stripe_begin, int32_t stripe_count, int64_t sink_slot,
                               hipStream_t stream) {
    if (n < 0) return fail(CPATTN_EINVAL, "n = %lld is negative", (long long)n);
    if (num_partners < 1 || interleave < 1 || page_size < 1 || page_size % num_partners ||
        (page_size / num_partners) % interleave)
        return fail(CPATTN_EINVAL, "num_partners * interleave = %lld must divide page_size = %d",
                    (long long)num_partners * interleave, page_size);
    if (stripe_count < 1 || stripe_begin < 0 || stripe_begin + stripe_count > num_partners)
        return fail(CPATTN_EINVAL, "stripes [%d, %d) outside [0, %d)", stripe_begin, stripe_begin + stripe_count,
                    num_partners);
    if (dtype != CPATTN_F32 && dtype != CPATTN_BF16 && dtype != CPATTN_FP8_E4M3)
        return fail(CPATTN_EINVAL, "dtype = %d unknown", dtype);
    if (num_kv_heads < 1 || head_dim < 1 || head_dim_v < 0 || num_pages < 1)
        return fail(CPATTN_EINVAL, "bad size (Hkv=%d, D=%d, Dv=%d, pages=%d)", num_kv_heads, head_dim, head_dim_v,
                    num_pages);
    if (src_stride_token < 0 || src_stride_head < 0 || kv_stride_stripe < 0 || kv_stride_page < 0 ||
        kv_stride_slot < 0 || kv_stride_head < 0)
        return fail(CPATTN_EINVAL, "negative stride");
    const int64_t pp = page_size / num_partners;
    if (sink_slot >= int64_t(num_pages) * pp)
        return fail(CPATTN_EINVAL, "sink_slot = %lld outside the pool", (long long)sink_slot);
    if (n == 0) return CPATTN_OK;
    if (!logical_slot || !k_src || !k_pool || (v_src && !v_pool)) return fail(CPATTN_EINVAL, "null pointer");
    const int64_t el = dtype == CPATTN_F32 ? 4 : dtype == CPATTN_BF16 ? 2 : 1;   // fp8 codes are copied as bytes
    KvWriteParams p{};
    p.slot = logical_slot;
    p.k_src = static_cast<const uint8_t*>(k_src);
    p.v_src = static_cast<const uint8_t*>(v_src);
    p.src_st = src_stride_token * el;
    p.src_sh = src_stride_head * el;
    p.kp = static_cast<uint8_t*>(k_pool);
    p.vp = static_cast<uint8_t*>(v_pool);
    p.s_stripe = kv_stride_stripe * el;
    p.s_page = kv_stride_page * el;
    p.s_slot = kv_stride_slot * el;
    p.s_head = kv_stride_head * el;
    p.n = n;
    p.P = num_partners;
    p.I = interleave;
    p.pp = pp;
    p.num_pages = num_pages;
    p.sink = sink_slot;
    p.stripe_begin = stripe_begin;
    p.stripe_count = stripe_count;
    p.Hkv = num_kv_heads;
    p.row_k_bytes = int32_t(head_dim * el);
    p.row_v_bytes = int32_t(head_dim_v * el);
    const int64_t blocks = n * stripe_count;
    if (blocks > (int64_t(1) << 31) - 1) return fail(CPATTN_EINVAL, "too many tokens for one call");
    hipLaunchKernelGGL(kv_write_kernel, dim3(uint32_t(blocks)), dim3(64), 0, stream, p);
    return check_launch("cp_kv_write");
}
