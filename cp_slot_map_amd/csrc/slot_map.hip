// cp_slot_map / cp_slot_map_rank: the write-addressing path of a context-parallel paged pool.
//
// Slot rule (mstar PR #1124, "Context / Sequence Parallel 1/5", PR description): the token in logical slot s is kept
// by partner s mod P at physical slot floor(s / P) of that partner's pool; page ids stay logical. Tokens of other
// partners go to the sink slot in the per-rank view. Negative slots (padding) are written nowhere.
#include "common.h"

namespace cpattn {

// One thread per slot; the divisor P is a runtime value, so the division is done once per element in 64-bit.
__global__ void slot_map_kernel(const int64_t* __restrict__ slot, int64_t n, int64_t P,
                                int32_t* __restrict__ partner, int64_t* __restrict__ phys) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t s = slot[i];
        if (s < 0) {
            partner[i] = -1;
            phys[i] = -1;
        } else {
            const int64_t q = s / P;
            partner[i] = int32_t(s - q * P);
            phys[i] = q;
        }
    }
}

__global__ void slot_map_rank_kernel(const int64_t* __restrict__ slot, int64_t n, int64_t P, int64_t rank,
                                     int64_t sink, int64_t* __restrict__ write_slot) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t s = slot[i];
        if (s < 0) {
            write_slot[i] = -1;
        } else {
            const int64_t q = s / P;
            write_slot[i] = (s - q * P) == rank ? q : sink;
        }
    }
}

static int32_t check_geometry(int64_t n, int32_t page_size, int32_t P) {
    if (n < 0) return fail(CPATTN_EINVAL, "n = %lld is negative", (long long)n);
    if (P < 1) return fail(CPATTN_EINVAL, "num_partners = %d must be >= 1", P);
    if (page_size < 1) return fail(CPATTN_EINVAL, "page_size = %d must be >= 1", page_size);
    if (page_size % P) return fail(CPATTN_EINVAL, "num_partners = %d must divide page_size = %d", P, page_size);
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
                               int32_t* partner_out, int64_t* phys_out, hipStream_t stream) {
    if (int32_t st = check_geometry(n, page_size, num_partners)) return st;
    if (n == 0) return CPATTN_OK;
    if (!logical_slot || !partner_out || !phys_out) return fail(CPATTN_EINVAL, "cp_slot_map: null pointer");
    hipLaunchKernelGGL(slot_map_kernel, grid_for(n), dim3(256), 0, stream, logical_slot, n, int64_t(num_partners),
                       partner_out, phys_out);
    return check_launch("cp_slot_map");
}

extern "C" int32_t cp_slot_map_rank(const int64_t* logical_slot, int64_t n, int32_t page_size, int32_t num_partners,
                                    int32_t rank, int64_t sink_slot, int64_t* write_slot_out, hipStream_t stream) {
    if (int32_t st = check_geometry(n, page_size, num_partners)) return st;
    if (rank < 0 || rank >= num_partners)
        return fail(CPATTN_EINVAL, "rank = %d outside [0, %d)", rank, num_partners);
    if (sink_slot < 0) return fail(CPATTN_EINVAL, "sink_slot = %lld is negative", (long long)sink_slot);
    if (n == 0) return CPATTN_OK;
    if (!logical_slot || !write_slot_out) return fail(CPATTN_EINVAL, "cp_slot_map_rank: null pointer");
    hipLaunchKernelGGL(slot_map_rank_kernel, grid_for(n), dim3(256), 0, stream, logical_slot, n,
                       int64_t(num_partners), int64_t(rank), sink_slot, write_slot_out);
    return check_launch("cp_slot_map_rank");
}
