// api.hip -- the C ABI declared in include/ggq.h: argument validation on the host,
// then one or more launches on the caller's stream.  Every check runs before any
// HIP call, so a rejected call enqueues nothing.
#include <limits.h>

#include <mutex>

#include "ggq.h"
#include "ggq_launch.h"

namespace {

constexpr int kMaxBatch = 16;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int block_of(int type) { return type == GGQ_Q8_0 ? 32 : (type == GGQ_Q4_K ? 256 : 0); }

int launched(hipError_t e) { return e == hipSuccess ? GGQ_OK : GGQ_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* ggq_status_string(int status) {
    switch (status) {
        case GGQ_OK: return "ok";
        case GGQ_ERR_ARG: return "invalid argument";
        case GGQ_ERR_UNSUPPORTED: return "unsupported format or mode";
        case GGQ_ERR_ALIGN: return "misaligned pointer or leading dimension";
        case GGQ_ERR_WORKSPACE: return "workspace missing or too small";
        case GGQ_ERR_LAUNCH: return "kernel launch failed";
        case GGQ_ERR_SCRATCH:
            return "call needs more than the fixed scratch of the no-allocation entry point";
        default: return "unknown status";
    }
}

int ggq_version(void) { return 100; }

int quant_dequantize(int type, const void* w, int64_t n, int64_t k, float* out, void* stream) {
    const int blk = block_of(type);
    if (!blk) return GGQ_ERR_UNSUPPORTED;
    if (n < 0 || k <= 0 || k % blk != 0) return GGQ_ERR_ARG;
    if (n == 0) return GGQ_OK;
    if (!w || !out) return GGQ_ERR_ARG;
    if (!aligned(w, 16) || !aligned(out, 16)) return GGQ_ERR_ALIGN;
    if (n * (k / 32) / 256 >= (int64_t)UINT_MAX) return GGQ_ERR_ARG;
    return launched(ggq::launch_dequant(type, static_cast<const uint8_t*>(w), n, k, out,
                                        as_stream(stream)));
}

namespace {
// Validation shared by quant_gemv and quant_gemv_grouped.  Tiles are counted in
// int32 inside the kernels: N is capped at 2^31 rows.
int check_gemv(int type, const ggq_gemv_desc& d, int batch) {
    const int blk = block_of(type);
    if (!blk) return GGQ_ERR_UNSUPPORTED;
    if (d.n < 0 || d.k <= 0 || d.k % blk != 0 || d.k > INT_MAX || d.n > INT_MAX)
        return GGQ_ERR_ARG;
    if (batch < 1 || batch > kMaxBatch) return GGQ_ERR_ARG;
    if (d.ldx < d.k || d.ldy < d.n) return GGQ_ERR_ARG;
    // Kernels address a matrix and an activation block with 32-bit buffer offsets.
    if ((d.n + 64) * ggq::row_bytes(type, d.k) >= ((int64_t)1 << 32) ||
        (int64_t)batch * d.ldx * 4 >= ((int64_t)1 << 32))
        return GGQ_ERR_ARG;
    if (d.n == 0) return GGQ_OK;
    if (!d.w || !d.x || !d.y) return GGQ_ERR_ARG;
    if (!aligned(d.w, 16) || !aligned(d.x, 16) || d.ldx % 4 != 0 || !aligned(d.y, 4))
        return GGQ_ERR_ALIGN;
    return GGQ_OK;
}
}  // namespace

// The matrix-core path needs rows that are whole 16-byte pieces (always true
// for Q4_K; K % 256 == 0 for Q8_0) and at least two activation rows.
static bool mfma_ok(int type, const ggq_gemv_desc* d, int count, int batch) {
    if (batch < 2) return false;
    for (int i = 0; i < count; ++i)
        if (d[i].n > 0 && type == GGQ_Q8_0 && d[i].k % 256 != 0) return false;
    return true;
}

// Workspace bytes (control block included) of the staged matrix-core path.
static size_t gemv_ws_need(int type, const ggq_gemv_desc* d, int count, int batch) {
    size_t need = ggq::kCtrlBytes;
    for (int i = 0; i < count; ++i)
        if (d[i].n > 0) need += ggq::gemv_mfma_ws_bytes(type, d[i].k, batch);
    return need;
}

static size_t gemv_split_need(int type, const ggq_gemv_desc* d, int count, int batch) {
    size_t need = ggq::kCtrlBytes;
    for (int i = 0; i < count; ++i)
        if (d[i].n > 0) need += ggq::gemv_split_ws_bytes(type, d[i].n, d[i].k, batch);
    if (count == 1 && d[0].n > 0) {
        const size_t ks = ggq::gemv_ks_ws_bytes(type, d[0].n, d[0].k, batch);
        need = ks > need ? ks : need;
    }
    return need;
}

static int run_gemv(int type, const ggq_gemv_desc* d, int count, int batch, void* ws,
                    size_t ws_bytes, void* stream) {
    if (ws) {
        if (!aligned(ws, 256)) return GGQ_ERR_ALIGN;
        if (ws_bytes < gemv_ws_need(type, d, count, batch)) return GGQ_ERR_WORKSPACE;
        // one matrix, batch >= 2: a single launch with the activation split done
        // in-kernel (at batch 1 the vector units' streaming kernel is faster,
        // except on Q4_K matrices of more than one round of workgroups)
        ggq::GemvKsPlan plan;
        if (count == 1 && ggq::gemv_ks_plan(type, d[0].n, d[0].k, batch, ws_bytes, plan) &&
            (batch >= 2 || plan.b1))
            return launched(ggq::launch_gemv_ks(type, d[0], batch, plan, ws, as_stream(stream)));
        const bool parts = ws_bytes >= gemv_split_need(type, d, count, batch);
        if (mfma_ok(type, d, count, batch))
            return launched(ggq::launch_gemv_mfma(type, d, count, batch,
                                                  static_cast<uint8_t*>(ws) + ggq::kCtrlBytes,
                                                  parts, as_stream(stream)));
    }
    return launched(ggq::launch_gemv_group(type, d, count, batch, as_stream(stream)));
}

int quant_gemv(int type, const void* w, int64_t n, int64_t k, const float* x, int64_t ldx,
               float* y, int64_t ldy, int batch, void* ws, size_t ws_bytes, void* stream) {
    const ggq_gemv_desc d{w, n, k, x, ldx, y, ldy};
    const int st = check_gemv(type, d, batch);
    if (st != GGQ_OK || n == 0) return st;
    return run_gemv(type, &d, 1, batch, ws, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// quant_gemv_noalloc: quant_gemv whose matrix-core workspace is a fixed array
// in device memory, for callers that cannot allocate.  Each device holds its
// own copy of `scratch` (allocated when the code object loads, kept until the
// process ends).  Host code never uses the array's name as an address: the
// device address is looked up once per device and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[GGQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Device address of `scratch` on the current device.
int scratch_of_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GGQ_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GGQ_ERR_LAUNCH;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GGQ_OK;
}
}  // namespace

extern "C" {

int quant_gemv_noalloc(int type, const void* w, int64_t n, int64_t k, const float* x,
                       int64_t ldx, float* y, int64_t ldy, int batch, void* stream) {
    const ggq_gemv_desc d{w, n, k, x, ldx, y, ldy};
    const int st = check_gemv(type, d, batch);
    if (st != GGQ_OK || n == 0) return st;
    // batch 1 (and Q8_0 rows that are not whole 256-column chunks) run on the
    // vector units, which use no workspace
    if (!mfma_ok(type, &d, 1, batch)) return run_gemv(type, &d, 1, batch, nullptr, 0, stream);
    const size_t need = gemv_ws_need(type, &d, 1, batch);
    if (need > (size_t)GGQ_NOALLOC_SCRATCH_BYTES) return GGQ_ERR_SCRATCH;
    void* sp = nullptr;
    const int rc = scratch_of_current_device(&sp);
    if (rc != GGQ_OK) return rc;
    // K parts (partial sums in the workspace) when their planes fit as well
    const size_t split = gemv_split_need(type, &d, 1, batch);
    return run_gemv(type, &d, 1, batch, sp,
                    split <= (size_t)GGQ_NOALLOC_SCRATCH_BYTES ? split : need, stream);
}

size_t quant_gemv_workspace_size(int type, int64_t k, int batch) {
    const int blk = block_of(type);
    if (!blk || k <= 0 || k % blk != 0 || batch < 1 || batch > kMaxBatch) return 0;
    return ggq::kCtrlBytes + ggq::gemv_mfma_ws_bytes(type, k, batch);
}

size_t quant_gemv_split_workspace_size(int type, int64_t n, int64_t k, int batch) {
    const size_t base = quant_gemv_workspace_size(type, k, batch);
    if (!base || n < 0 || n > INT_MAX) return 0;
    const size_t old = ggq::kCtrlBytes + ggq::gemv_split_ws_bytes(type, n, k, batch);
    const size_t ks = n > 0 ? ggq::gemv_ks_ws_bytes(type, n, k, batch) : 0;
    return ks > old ? ks : old;
}

int quant_gemv_grouped(int type, const ggq_gemv_desc* descs, int count, int batch, void* ws,
                       size_t ws_bytes, void* stream) {
    if (!block_of(type)) return GGQ_ERR_UNSUPPORTED;
    if (!descs || count < 1 || count > ggq::gemv_max_group()) return GGQ_ERR_ARG;
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) {
        const int st = check_gemv(type, descs[i], batch);
        if (st != GGQ_OK) return st;
        tiles += (descs[i].n + 7) / 8;
    }
    if (tiles > INT_MAX) return GGQ_ERR_ARG;
    if (tiles == 0) return GGQ_OK;
    return run_gemv(type, descs, count, batch, ws, ws_bytes, stream);
}

// Up to 16 rows the GEMM runs as the batched decode GEMV (one read of W, no
// padding of M to the GEMM's row tiles); its workspace must fit either path.
constexpr int64_t kGemmViaGemvRows = 16;

static size_t gemm_ws_need(int type, int64_t m, int64_t n, int64_t k) {
    size_t need = ggq::kCtrlBytes + ggq::gemm_workspace_bytes(type, m, n, k);
    if (m >= 1 && m <= kGemmViaGemvRows) {
        const ggq_gemv_desc d{nullptr, n, k, nullptr, k, nullptr, n};
        const size_t g = gemv_split_need(type, &d, 1, (int)m);
        need = g > need ? g : need;
    }
    return need;
}

int quant_gemv_swiglu(int type, const void* wg, const void* wu, int64_t n, int64_t k,
                      const float* x, int64_t ldx, float* h, int64_t ldh, int batch, void* ws,
                      size_t ws_bytes, void* stream) {
    if (!block_of(type)) return GGQ_ERR_UNSUPPORTED;
    const ggq_gemv_desc dg{wg, n, k, x, ldx, h, ldh}, du{wu, n, k, x, ldx, h, ldh};
    int st = check_gemv(type, dg, batch);
    if (st == GGQ_OK) st = check_gemv(type, du, batch);
    if (st != GGQ_OK) return st;
    if (k % 256 != 0) return GGQ_ERR_ARG;
    if (n == 0) return GGQ_OK;
    if (batch >= 2) {
        if (!ws || ws_bytes < ggq::kCtrlBytes + ggq::gemv_mfma_ws_bytes(type, k, batch))
            return GGQ_ERR_WORKSPACE;
        if (!aligned(ws, 256)) return GGQ_ERR_ALIGN;
        ws = static_cast<uint8_t*>(ws) + ggq::kCtrlBytes;
    }
    return launched(ggq::launch_swiglu(type, static_cast<const uint8_t*>(wg),
                                       static_cast<const uint8_t*>(wu), n, k, x, ldx, h, ldh,
                                       batch, ws, as_stream(stream)));
}

size_t quant_gemm_workspace_size(int type, int64_t m, int64_t n, int64_t k, int mode) {
    const int blk = block_of(type);
    if (!blk || mode != GGQ_GEMM_BF16 || m < 0 || n < 0 || k <= 0 || k % blk != 0) return 0;
    if (n > (int64_t)INT_MAX || m > (int64_t)INT_MAX) return 0;
    return gemm_ws_need(type, m, n, k);
}

int quant_gemm(int type, const void* w, int64_t n, int64_t k, const float* a, int64_t lda,
               int64_t m, float* c, int64_t ldc, int mode, void* ws, size_t ws_bytes,
               void* stream) {
    const int blk = block_of(type);
    if (!blk || mode != GGQ_GEMM_BF16) return GGQ_ERR_UNSUPPORTED;
    if (n < 0 || m < 0 || k <= 0 || k % blk != 0 || lda < k || ldc < n) return GGQ_ERR_ARG;
    if (n > (int64_t)INT_MAX || m > (int64_t)INT_MAX) return GGQ_ERR_ARG;
    // the bf16 copy of A is addressed with 32-bit buffer offsets
    if ((m + 15) / 16 * 16 * ((k + 255) / 256 * 256) * 2 >= ((int64_t)1 << 31)) return GGQ_ERR_ARG;
    // ... and so are the weight blocks
    if (n * ggq::row_bytes(type, k) >= ((int64_t)1 << 32)) return GGQ_ERR_ARG;
    if (m == 0 || n == 0) return GGQ_OK;
    if (!w || !a || !c) return GGQ_ERR_ARG;
    if (!aligned(w, 16) || !aligned(a, 16) || lda % 4 != 0 || !aligned(c, 4)) return GGQ_ERR_ALIGN;
    if (!ws || ws_bytes < gemm_ws_need(type, m, n, k)) return GGQ_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return GGQ_ERR_ALIGN;
    if (m <= kGemmViaGemvRows) {
        const ggq_gemv_desc d{w, n, k, a, lda, c, ldc};
        if (check_gemv(type, d, (int)m) == GGQ_OK)
            return run_gemv(type, &d, 1, (int)m, ws, ws_bytes, stream);
    }
    return launched(ggq::launch_gemm(type, static_cast<const uint8_t*>(w), n, k, a, lda, m, c, ldc,
                                     static_cast<uint8_t*>(ws) + ggq::kCtrlBytes,
                                     as_stream(stream)));
}

int moe_route(const float* wr, int64_t e, int64_t h, const float* x, int64_t t, int top_k,
              int32_t* idx, float* probs, float* logits, void* stream) {
    if (e < 1 || e > kMaxExperts || h < 4 || h % 4 != 0 || h > (1 << 24) || t < 0) return GGQ_ERR_ARG;
    if (top_k < 1 || top_k > kMaxTopK || top_k > e) return GGQ_ERR_ARG;
    if (t > INT_MAX) return GGQ_ERR_ARG;
    if (t == 0) return GGQ_OK;
    if (!wr || !x || !idx || !probs || !logits) return GGQ_ERR_ARG;
    if (!aligned(wr, 16) || !aligned(x, 16) || !aligned(idx, 4) || !aligned(probs, 4) ||
        !aligned(logits, 4))
        return GGQ_ERR_ALIGN;
    return launched(ggq::launch_route(wr, e, h, x, t, top_k, idx, probs, logits, as_stream(stream)));
}

size_t moe_workspace_size(int64_t e, int64_t t, int top_k, int64_t h, int64_t f) {
    if (e < 1 || e > kMaxExperts || t < 1 || top_k < 1 || top_k > kMaxTopK || h < 1 || f < 1)
        return 0;
    return ggq::moe_ws_bytes(e, t, top_k, h, f);
}

size_t moe_workspace_h_offset(int64_t e, int64_t t, int top_k) {
    if (e < 1 || t < 1 || top_k < 1) return 0;
    return ggq::moe_ws_h_offset(e, t, top_k);
}

// Arguments shared by the two expert feed-forward entry points.
static int check_moe(int type, const void* wg, const void* wu, const void* wd, int64_t e, int64_t h,
                     int64_t f, const float* x, int64_t t, const int32_t* idx, const float* probs,
                     int top_k, float* y) {
    if (!block_of(type)) return GGQ_ERR_UNSUPPORTED;
    if (e < 1 || e > kMaxExperts || t < 0 || top_k < 1 || top_k > kMaxTopK || top_k > e)
        return GGQ_ERR_ARG;
    if (h < 256 || f < 256 || h % 256 != 0 || f % 256 != 0 || h > INT_MAX || f > INT_MAX)
        return GGQ_ERR_ARG;
    if (t * top_k > 65536) return GGQ_ERR_ARG;
    if (t == 0) return GGQ_OK;
    if (!wg || !wu || !wd || !x || !idx || !probs || !y) return GGQ_ERR_ARG;
    if (!aligned(wg, 16) || !aligned(wu, 16) || !aligned(wd, 16) || !aligned(x, 16) ||
        !aligned(y, 4) || !aligned(idx, 4) || !aligned(probs, 4))
        return GGQ_ERR_ALIGN;
    // one expert's matrix is addressed with 32-bit buffer offsets
    if (f * ggq::row_bytes(type, h) >= ((int64_t)1 << 32) ||
        h * ggq::row_bytes(type, f) >= ((int64_t)1 << 32))
        return GGQ_ERR_ARG;
    return GGQ_OK;
}

int moe_expert_gemv(int type, const void* wg, const void* wu, const void* wd, int64_t e,
                    int64_t h, int64_t f, const float* x, int64_t t, const int32_t* idx,
                    const float* probs, int top_k, float* y, void* ws, size_t ws_bytes,
                    void* stream) {
    const int rc = check_moe(type, wg, wu, wd, e, h, f, x, t, idx, probs, top_k, y);
    if (rc != GGQ_OK || t == 0) return rc;
    // the stages address x [T][H], h [T*top_k][F] and the per-slot down
    // outputs [T*top_k][H] with 32-bit buffer offsets
    const int64_t lim = (int64_t)1 << 32;
    if (t * h * 4 >= lim || t * top_k * f * 4 >= lim || t * top_k * h * 4 >= lim)
        return GGQ_ERR_ARG;
    if (!ws || ws_bytes < ggq::moe_ws_bytes(e, t, top_k, h, f)) return GGQ_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return GGQ_ERR_ALIGN;
    return launched(ggq::launch_moe(type, static_cast<const uint8_t*>(wg),
                                    static_cast<const uint8_t*>(wu),
                                    static_cast<const uint8_t*>(wd), e, h, f, x, t, idx, probs,
                                    top_k, y, ws, as_stream(stream)));
}

size_t moe_layer_workspace_size(int64_t e, int64_t t, int top_k, int64_t h, int64_t f) {
    if (e < 1 || e > kMaxExperts || t < 1 || top_k < 1 || top_k > kMaxTopK || h < 1 || f < 1)
        return 0;
    return ggq::moe_layer_ws_bytes(e, t, top_k, h, f);
}

int moe_layer_gemv(int type, const float* wr, const void* wg, const void* wu, const void* wd,
                   int64_t e, int64_t h, int64_t f, const float* x, int64_t t, int top_k,
                   float* logits, int32_t* idx, float* probs, float* y, void* ws, size_t ws_bytes,
                   void* stream) {
    // the arguments of moe_route and of moe_expert_gemv
    if (h > (1 << 24) || t > INT_MAX) return GGQ_ERR_ARG;
    const int rc = check_moe(type, wg, wu, wd, e, h, f, x, t, idx, probs, top_k, y);
    if (rc != GGQ_OK || t == 0) return rc;
    if (!wr || !logits) return GGQ_ERR_ARG;
    if (!aligned(wr, 16) || !aligned(logits, 4)) return GGQ_ERR_ALIGN;
    const int64_t lim = (int64_t)1 << 32;
    if (t * h * 4 >= lim || t * top_k * f * 4 >= lim || t * top_k * h * 4 >= lim)
        return GGQ_ERR_ARG;
    if (!ws || ws_bytes < ggq::moe_layer_ws_bytes(e, t, top_k, h, f)) return GGQ_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return GGQ_ERR_ALIGN;
    return launched(ggq::launch_moe_layer(type, wr, static_cast<const uint8_t*>(wg),
                                          static_cast<const uint8_t*>(wu),
                                          static_cast<const uint8_t*>(wd), e, h, f, x, t, top_k,
                                          logits, idx, probs, y, ws, as_stream(stream)));
}

size_t moe_gemm_workspace_size(int64_t e, int64_t t, int top_k, int64_t h, int64_t f) {
    if (e < 1 || e > kMaxExperts || t < 1 || top_k < 1 || top_k > kMaxTopK || h < 1 || f < 1)
        return 0;
    if (t * top_k > 65536) return 0;
    return ggq::moe_gemm_ws_bytes(e, t, top_k, h, f);
}

int moe_expert_gemm(int type, const void* wg, const void* wu, const void* wd, int64_t e,
                    int64_t h, int64_t f, const float* x, int64_t t, const int32_t* idx,
                    const float* probs, int top_k, float* y, void* ws, size_t ws_bytes,
                    void* stream) {
    const int rc = check_moe(type, wg, wu, wd, e, h, f, x, t, idx, probs, top_k, y);
    if (rc != GGQ_OK || t == 0) return rc;
    // bf16 x and h are addressed with 31-bit buffer offsets
    const int64_t slots = ggq::moe_gemm_slot_bound(e, t * top_k);
    if (t * h * 2 >= ((int64_t)1 << 31) || slots * f * 2 >= ((int64_t)1 << 31)) return GGQ_ERR_ARG;
    if (!ws || ws_bytes < ggq::moe_gemm_ws_bytes(e, t, top_k, h, f)) return GGQ_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return GGQ_ERR_ALIGN;
    return launched(ggq::launch_moe_gemm(type, static_cast<const uint8_t*>(wg),
                                         static_cast<const uint8_t*>(wu),
                                         static_cast<const uint8_t*>(wd), e, h, f, x, t, idx,
                                         probs, top_k, y, ws, as_stream(stream)));
}

}  // extern "C"
