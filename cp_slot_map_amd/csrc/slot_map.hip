// cp_slot_map / cp_slot_map_rank: the write-addressing path of a context-parallel paged pool.
//
// Slot rule (mstar PR #1124, "Context / Sequence Parallel 1/5", PR description): the token in logical slot s is kept
// by partner s mod P at physical slot floor(s / P) of that partner's pool; page ids stay logical. Tokens of other
// partners go to the sink slot in the per-rank view. Negative slots (padding) are written nowhere. With a KV-cache
// interleave size I (read from the parallel config in the vLLM compare view "[Core] Add explicit layer parallel
// plans"; placement is our reading) runs of I consecutive slots go to one partner, partners in turn: partner
// floor(s / I) mod P, physical slot floor(s / (I P)) * I + s mod I. I = 1 is the PR's rule.
#include "common.h"

namespace cpattn {

// One thread per slot; the divisor P is a runtime value, so the division is done once per element in 64-bit.
__global__ void slot_map_kernel(const int64_t* __restrict__ slot, int64_t n, int64_t P, int64_t I,
                                int32_t* __restrict__ partner, int64_t* __restrict__ phys) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t s = slot[i];
        if (s < 0) {
            partner[i] = -1;
            phys[i] = -1;
        } else {
            int32_t a;
            int64_t b;
            place_slot(s, P, I, a, b);
            partner[i] = a;
            phys[i] = b;
        }
    }
}

__global__ void slot_map_rank_kernel(const int64_t* __restrict__ slot, int64_t n, int64_t P, int64_t I, int64_t rank,
                                     int64_t sink, int64_t* __restrict__ write_slot) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t s = slot[i];
        if (s < 0) {
            write_slot[i] = -1;
        } else {
            int32_t a;
            int64_t b;
            place_slot(s, P, I, a, b);
            write_slot[i] = a == rank ? b : sink;
        }
    }
}

static int32_t check_geometry(int64_t n, int32_t page_size, int32_t P, int32_t I) {
    if (n < 0) return fail(CPATTN_EINVAL, "n = %lld is negative", (long long)n);
    if (P < 1) return fail(CPATTN_EINVAL, "num_partners = %d must be >= 1", P);
    if (I < 1) return fail(CPATTN_EINVAL, "interleave = %d must be >= 1", I);
    if (page_size < 1) return fail(CPATTN_EINVAL, "page_size = %d must be >= 1", page_size);
    if (page_size % P || (page_size / P) % I)
        return fail(CPATTN_EINVAL, "num_partners * interleave = %lld must divide page_size = %d", (long long)P * I,
                    page_size);
    return CPATTN_OK;
}

static dim3 grid_for(int64_t n) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return dim3(uint32_t(blocks));
}

}  // namespace cpattn

using namespace cpattn;

extern "C" int32_t cp_slot_map(const int64_t* logical_slot, int64_t n, int32_t page_size, int32_t num_partners,
                               int32_t interleave, int32_t* partner_out, int64_t* phys_out, hipStream_t stream) {
    if (int32_t st = check_geometry(n, page_size, num_partners, interleave)) return st;
    if (n == 0) return CPATTN_OK;
    if (!logical_slot || !partner_out || !phys_out) return fail(CPATTN_EINVAL, "cp_slot_map: null pointer");
    hipLaunchKernelGGL(slot_map_kernel, grid_for(n), dim3(256), 0, stream, logical_slot, n, int64_t(num_partners),
                       int64_t(interleave), partner_out, phys_out);
    return check_launch("cp_slot_map");
}

extern "C" int32_t cp_slot_map_rank(const int64_t* logical_slot, int64_t n, int32_t page_size, int32_t num_partners,
                                    int32_t interleave, int32_t rank, int64_t sink_slot, int64_t* write_slot_out,
                                    hipStream_t stream) {
    if (int32_t st = check_geometry(n, page_size, num_partners, interleave)) return st;
    if (rank < 0 || rank >= num_partners)
        return fail(CPATTN_EINVAL, "rank = %d outside [0, %d)", rank, num_partners);
    if (sink_slot < 0) return fail(CPATTN_EINVAL, "sink_slot = %lld is negative", (long long)sink_slot);
    if (n == 0) return CPATTN_OK;
    if (!logical_slot || !write_slot_out) return fail(CPATTN_EINVAL, "cp_slot_map_rank: null pointer");
    hipLaunchKernelGGL(slot_map_rank_kernel, grid_for(n), dim3(256), 0, stream, logical_slot, n,
                       int64_t(num_partners), int64_t(interleave), int64_t(rank), sink_slot, write_slot_out);
    return check_launch("cp_slot_map_rank");
}
