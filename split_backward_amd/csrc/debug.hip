// Debug aids of the stage: ring-slot tags checked on the device, in stream
// order with the passes.
//
// The ring reuses a slot only after the W that read it has run (the
// pages' "Memory Management & Activation Rollback" frees a microbatch's
// stash when its W is done); the host enforces that order with events.  The
// tags check, on the device, that every pass finds its slot in the state
// that order implies when the pass actually runs:
//   tag = 4 * mb + phase   (phase 1: F done, 2: B done, 3: W done)
//   tag = -1               (never used since the tags were reset)
// F(mb) needs a free slot (-1 or phase 3), B(mb) needs 4 mb + 1 and W(mb)
// needs 4 mb + 2.  A mismatch is counted and recorded, never trapped.
#include "common.h"

namespace zb {
namespace {

// Single-lane check-and-set.  Plain loads and vector stores: the two
// streams of a replay never touch one slot's tag at the same time unless
// the ordering under test is broken, and then a lost count still leaves it
// non-zero.
__global__ void slot_tag_kernel(int32_t* tags, int32_t* rec, int slot, int op, int mb, int expect, int set) {
    if (threadIdx.x != 0) return;
    volatile int32_t* t = tags + slot;
    const int32_t cur = *t;
    bool ok = true;
    if (expect == TAG_FREE) ok = cur < 0 || (cur & 3) == 3;
    else if (expect != TAG_ANY) ok = cur == expect;
    if (!ok) {
        volatile int32_t* r = rec;
        r[0] = r[0] + 1;
        r[1] = op;
        r[2] = mb;
        r[3] = slot;
        r[4] = cur;
        r[5] = expect;
    }
    if (set != TAG_KEEP) *t = set;
}

__global__ void tag_reset_kernel(int32_t* tags, int n, int32_t* rec) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) tags[i] = -1;
    if (threadIdx.x < DEBUG_REC) rec[threadIdx.x] = 0;
}

}  // namespace

int32_t slot_tag(int32_t* tags, int32_t* rec, int slot, int op, int mb, int expect, int set, hipStream_t s) {
    hipLaunchKernelGGL(slot_tag_kernel, dim3(1), dim3(64), 0, s, tags, rec, slot, op, mb, expect, set);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

int32_t tag_reset(int32_t* tags, int n, int32_t* rec, hipStream_t s) {
    hipLaunchKernelGGL(tag_reset_kernel, dim3(1), dim3(256), 0, s, tags, n, rec);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

}  // namespace zb
