// ggq_launch.h -- host-side launchers behind the C ABI (internal).
// Arguments reaching these functions have already been validated by api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ggq.h"

namespace ggq {

using GemvDesc = ggq_gemv_desc;

// Every quant_gemv / quant_gemm workspace begins with a control block: the
// per-row-tile counters of the single-launch GEMV (gemv_ks.hip).  It must be
// zero before a workspace is first used; every call leaves it zero.  The other
// layouts start after it, so one workspace can serve all of these calls.
constexpr size_t kCtrlBytes = 4096;

int64_t row_bytes(int type, int64_t k);

hipError_t launch_dequant(int type, const uint8_t* w, int64_t n, int64_t k, float* out,
                          hipStream_t s);

int gemv_max_group();
size_t gemv_mfma_ws_bytes(int type, int64_t k, int batch);
// With room for partial sums after each job's region, K may be cut into more
// than two parts per tile (`parts`).
size_t gemv_split_ws_bytes(int type, int64_t n, int64_t k, int batch);
hipError_t launch_gemv_mfma(int type, const GemvDesc* descs, int count, int batch, void* ws,
                            bool parts, hipStream_t s);
hipError_t launch_gemv_group(int type, const GemvDesc* descs, int count, int batch, hipStream_t s);
hipError_t launch_gemv(int type, const uint8_t* w, int64_t n, int64_t k, const float* x,
                       int64_t ldx, float* y, int64_t ldy, int batch, hipStream_t s);

// One-launch matrix-core GEMV for a single matrix (gemv_ks.hip): the plan, or
// false when the shape or the workspace does not suit it.
struct GemvKsPlan {
    int t, mt, tiles, parts;
    size_t ws_bytes;   // workspace the plan needs (0 without K parts)
    bool b1;           // also faster than the vector-unit kernel at batch 1
};
bool gemv_ks_plan(int type, int64_t n, int64_t k, int batch, size_t ws_bytes, GemvKsPlan& p);
size_t gemv_ks_ws_bytes(int type, int64_t n, int64_t k, int batch);
hipError_t launch_gemv_ks(int type, const GemvDesc& d, int batch, const GemvKsPlan& p, void* ws,
                          hipStream_t s);

// Workspace layout of the prompt GEMM.
size_t gemm_workspace_bytes(int type, int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm(int type, const uint8_t* w, int64_t n, int64_t k, const float* a,
                       int64_t lda, int64_t m, float* c, int64_t ldc, void* ws, hipStream_t s);

hipError_t launch_route(const float* wr, int64_t e, int64_t h, const float* x, int64_t t,
                        int top_k, int32_t* idx, float* probs, float* logits, hipStream_t s);

hipError_t launch_swiglu(int type, const uint8_t* wg, const uint8_t* wu, int64_t n, int64_t k,
                         const float* x, int64_t ldx, float* h, int64_t ldh, int batch, void* ws,
                         hipStream_t s);

size_t moe_ws_bytes(int64_t e, int64_t t, int top_k, int64_t h, int64_t f);
size_t moe_ws_h_offset(int64_t e, int64_t t, int top_k);
hipError_t launch_moe(int type, const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
                      int64_t e, int64_t h, int64_t f, const float* x, int64_t t,
                      const int32_t* idx, const float* probs, int top_k, float* y, void* ws,
                      hipStream_t s);

// moe_route then moe_expert_gemv; one token: the router and the selection in
// one launch.  Workspace: the control block, then the moe_expert_gemv workspace.
size_t moe_layer_ws_bytes(int64_t e, int64_t t, int top_k, int64_t h, int64_t f);
hipError_t launch_moe_layer(int type, const float* wr, const uint8_t* wg, const uint8_t* wu,
                            const uint8_t* wd, int64_t e, int64_t h, int64_t f, const float* x,
                            int64_t t, int top_k, float* logits, int32_t* idx, float* probs,
                            float* y, void* ws, hipStream_t s);

// y[t] = sum_s probs[t][s] * dbuf[t*top_k + s] (slot order; out-of-range experts count 0).
hipError_t launch_combine(const float* dbuf, const int32_t* idx, const float* probs, int64_t e,
                          int64_t h, int64_t t, int top_k, float* y, hipStream_t s);

// quant_gemm for 17..kGemmMidRows rows (moe_gemm.hip's grouped tile as a dense
// product), where it covers the device; A goes to bf16 at the start of ws.
constexpr int64_t kGemmMidRows = 128;
bool gemm_mid_applies(int type, int64_t m, int64_t n, int64_t k);
size_t gemm_mid_ws_bytes(int64_t m, int64_t k);
hipError_t launch_gemm_mid(int type, const uint8_t* w, int64_t n, int64_t k, const float* a,
                           int64_t lda, int64_t m, float* c, int64_t ldc, void* ws, hipStream_t s);

// Routed expert feed-forward at prompt batch (grouped matrix-core GEMMs).
int64_t moe_gemm_slot_bound(int64_t e, int64_t p);
int64_t moe_gemm_tile_bound(int64_t e, int64_t p);
size_t moe_gemm_ws_bytes(int64_t e, int64_t t, int top_k, int64_t h, int64_t f);
hipError_t launch_moe_gemm(int type, const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
                           int64_t e, int64_t h, int64_t f, const float* x, int64_t t,
                           const int32_t* idx, const float* probs, int top_k, float* y, void* ws,
                           hipStream_t s);

}  // namespace ggq
