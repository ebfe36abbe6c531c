// Internal definition of the stage object shared by the C ABI, the passes
// and the executor.
#pragma once

#include <array>
#include <vector>

#include "common.h"

namespace zb {

constexpr int MAX_RUN_OPS = 4096;  // executor stamp capacity (ops per run)

// Stash tensor indices (the "which" argument of zb_stage_stash_tensor).
enum { LIN_X = 0, LIN_DY = 1 };
enum { MLP_X = 0, MLP_A = 1, MLP_H = 2, MLP_DY = 3, MLP_DA = 4 };
enum {
    L_X = 0, L_R1, L_N1, L_QKV, L_A, L_LSE, L_H1, L_R2, L_N2, L_GU, L_S,  // kept by F
    L_DOUT, L_DGU, L_DN2, L_DH1, L_DQKV, L_DN1,                           // kept by B
    // ZB_FP8 stages: the W-only operands as transposed E4M3 codes
    // ([features][tokens]) and their exponents (int32, in this order);
    // those stages keep no bf16 n1, n2, s, dout, dgu, dh1, dqkv.
    L_N1T, L_AT, L_N2T, L_ST, L_DOUTT, L_DGUT, L_DH1T, L_DQKVT, L_QEXP
};
constexpr int NQ8 = 8;  // quantized stash tensors per layer (L_N1T .. L_DQKVT)
enum { PASS_F = 0, PASS_B = 1, PASS_W = 2 };

struct Layout {
    struct Tensor {
        int layer, which, rows, cols, dtype;
        size_t offset;  // within a slot
    };
    std::vector<Tensor> off;
    size_t slot_bytes = 0, ring_bytes = 0, scratch_b = 0, scratch_w = 0, stamps_bytes = 0, debug_bytes = 0, total = 0;
    // ZB_FP8 stages: F-pass scratch, the E4M3 weight copies, and offsets
    // inside the pass scratch (bytes from its start).
    size_t scratch_f = 0, w8_bytes = 0;
    size_t f_act = 0, f_q = 0, f_part = 0;                                  // F scratch
    size_t b_dgu = 0, b_dh1 = 0, b_dqkv = 0, b_dout[2] = {0, 0}, b_q = 0, b_part = 0;  // B scratch
    // floats of partial maxima at f_part and b_part (the amax pass's, one per
    // row of an RMSNorm, or one per wave of a SwiGLU GEMM launch), followed
    // by the one float they reduce to
    size_t amax_cap = 0;
    std::vector<size_t> w8_q, w8_qt, w8_e;                                  // per weight index (0 if none)
    // bf16 Llama stages: transposed copies [in][out] of the linear weights,
    // which the B pass reads so that its products have both operands
    // K-contiguous (offset per weight index, 0 for the norm gains).
    size_t wt_bytes = 0;
    std::vector<size_t> wt_off;
    void build(const zb_stage_desc& d);
    const Tensor* find(int layer, int which) const;
};

struct Slot {
    int mb = -1;  // resident microbatch, -1 = free
    bool b_issued = false, w_issued = false;
    bool w_event_valid = false;  // evW was recorded at least once
    hipEvent_t evF = nullptr, evB = nullptr, evW = nullptr;
};

size_t weight_elems(const zb_stage_desc& d, int i);

}  // namespace zb

struct zb_stage {
    zb_stage_desc desc{};
    zb::Layout lay;
    std::vector<void*> w;
    std::vector<float*> dw;
    char* ws = nullptr;
    char* scratch_b = nullptr;
    char* scratch_w = nullptr;
    char* scratch_f = nullptr;  // ZB_FP8: F-pass scratch
    char* w8 = nullptr;         // ZB_FP8: E4M3 weight copies
    bool w8_dirty = true;       // ZB_FP8: refresh the copies at the next F
    char* wt = nullptr;         // bf16 ZB_LLAMA: transposed weight copies
    bool wt_dirty = true;       // bf16 ZB_LLAMA: refresh them at the next B
    uint64_t* stamps = nullptr;
    std::vector<zb::Slot> slots;
    std::array<hipEvent_t, 3> chain{};     // last op of each pass (scratch reuse order)
    std::array<bool, 3> chain_valid{};
    int next_f = 0, next_w = 0;
    float lr = 0.f;  // learning rate of the executor's optimizer-step ops
    int device = 0;  // the HIP device current when the stage was created
    // Debug aids (zb_stage_set_debug): flags, the injected delay before each
    // W pass, and the workspace's debug area (ring-slot tags, the mismatch
    // record, the delay's clock stamp).
    int debug_flags = 0;
    int w_delay_us = 0;
    int32_t* tags = nullptr;
    int32_t* dbg_rec = nullptr;
    uint64_t* dbg_t0 = nullptr;

    ~zb_stage();
    void* slot_tensor(int mb, int layer, int which) const;
    int32_t order_after(int pass, hipEvent_t dep, bool dep_valid, hipStream_t s);
    int32_t finish(int pass, hipEvent_t ev, hipStream_t s);
    // Make `s` wait for every event the op (type, mb) waits for when it is
    // issued (its pass's previous op, the microbatch's previous op, and for F
    // the W that frees its ring slot); issues nothing for an op that its own
    // call would reject.  The executor calls this before an op's start stamp,
    // so the stamp marks the moment the op can actually run.
    int32_t wait_deps(int type, int mb, hipStream_t s);
    // Debug hooks of the passes; each does nothing unless its flag is set.
    // tag: check-and-set of the slot tag of microbatch mb (slot_tag).
    int32_t tag(int op, int mb, int expect, int set, hipStream_t s);
    // Before a W pass: wait w_delay_us on the device.
    int32_t delay_w(hipStream_t s);
    // After every op: wait for the whole device and report its errors.
    int32_t serialize();
};

namespace zb {
int32_t run_forward(zb_stage& st, int mb, const void* x, void* y, hipStream_t s);
int32_t run_backward_input(zb_stage& st, int mb, const void* dy, void* dx, hipStream_t s);
// dg_part: fp32 scratch of the RMSNorm dgamma partials
// (dgamma_scratch_bytes); nullptr = the stage's workspace scratch.
int32_t run_backward_weight(zb_stage& st, int mb, hipStream_t s, float* dg_part = nullptr);
size_t dgamma_scratch_bytes(const zb_stage_desc& d);
// zb_bwd_weight_accum with the dgamma partials in dg_part (nullptr: the
// stage's workspace scratch).
int32_t bwd_weight_accum(zb_stage* st, int mb, hipStream_t s, float* dg_part);
int32_t run_backward_weight_pair(zb_stage& st, int mb, hipStream_t s);
// ZB_FP8 Llama stages (passes_fp8.cpp)
int32_t run_forward_fp8(zb_stage& st, int mb, const void* x, void* y, hipStream_t s);
int32_t run_backward_input_fp8(zb_stage& st, int mb, const void* dy, void* dx, hipStream_t s);
int32_t run_backward_weight_fp8(zb_stage& st, int mb, hipStream_t s, float* dg_part);
// bf16 Llama stages: write the transposed weight copies (passes.cpp).
int32_t transpose_weights(zb_stage& st, hipStream_t s);
}  // namespace zb
