// W for one microbatch with no scratch memory from the caller or the
// library's workspace: for callers that cannot allocate (code under HIP graph
// capture, tight loops, harnesses that forbid allocation).
//
// The only scratch of the W pass is the fp32 partial sums of the RMSNorm gain
// gradients (one row of `hidden` floats per 64-token chunk of the
// microbatch).  Here they live in `scratch`, a file-scope device array of
// fixed size that every GPU the library runs on holds until the process
// ends.  Host code never uses the array's name as an address: the device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept in `dev_scratch`.  Every call on a GPU shares that
// GPU's array, so calls that overlap in time on one GPU (two stages, or two
// streams without ordering between them) race; the partials kernel writes
// every value the reduction then reads, so nothing needs clearing between
// calls.
#include <mutex>
#include <string>

#include "common.h"
#include "stage.h"

namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(8) << 20;  // ZB_NOALLOC_SCRATCH_BYTES
static_assert(NOALLOC_SCRATCH_BYTES == ZB_NOALLOC_SCRATCH_BYTES, "zb.h and the array must agree");

__device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex dev_mu;
void* dev_scratch[MAX_DEVICES];

// Device address of `scratch` on `dev`, which must be the current device.
int32_t scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= MAX_DEVICES) return zb::fail(ZB_EINVAL, "zb_bwd_weight_accum_noalloc: device index out of range");
    std::lock_guard<std::mutex> lock(dev_mu);
    if (!dev_scratch[dev]) {
        void* p = nullptr;
        ZB_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return zb::fail(ZB_EHIP, "zb_bwd_weight_accum_noalloc: no device address for the scratch array");
        dev_scratch[dev] = p;
    }
    *out = dev_scratch[dev];
    return ZB_OK;
}

}  // namespace

extern "C" int32_t zb_bwd_weight_accum_noalloc(zb_stage* st, int32_t mb, void* stream) {
    if (!st || mb < 0) return zb::fail(ZB_EINVAL, "zb_bwd_weight_accum_noalloc: bad argument");
    const size_t need = zb::dgamma_scratch_bytes(st->desc);
    if (need > NOALLOC_SCRATCH_BYTES)
        return zb::fail(ZB_EINVAL, "zb_bwd_weight_accum_noalloc: the stage needs " + std::to_string(need) +
                                       " bytes of dgamma scratch, more than the fixed " +
                                       std::to_string(NOALLOC_SCRATCH_BYTES) +
                                       " (tokens/64 rounded up, times hidden, times 4 bytes)");
    int dev = -1;
    ZB_HIP(hipGetDevice(&dev));
    if (dev != st->device)
        return zb::fail(ZB_EINVAL, "zb_bwd_weight_accum_noalloc: make the stage's device (" +
                                       std::to_string(st->device) + ") current");
    void* p = nullptr;
    const int32_t rc = scratch_address(dev, &p);
    if (rc) return rc;
    return zb::bwd_weight_accum(st, mb, static_cast<hipStream_t>(stream), static_cast<float*>(p));
}
