// moe.hip -- router/top-k (moe_route) and the routed expert feed-forward
// (moe_expert_gemv) of a mixture-of-experts layer.
//
// Phobos README, opening paragraph: each token of a mixture-of-experts model is
// sent to a few experts and only those experts' weights take part (the README's
// engine caches experts on the card; here every expert is resident in HBM and
// the selection becomes an expert-indexed gather).
//
// Router: logits = Wr x (fp32), top_k by logit in rank order with equal logits
// ranking the lower expert index first (softmax is increasing in the logit, so
// this is the top_k by probability), probabilities renormalised over the
// selected set.
//
// Expert layer, four launches on the caller's stream:
//   1. group   : one workgroup sorts the T*top_k (token, slot) pairs by expert
//                (stable), giving per-expert pair lists and the ascending list
//                of experts that received any pair.
//   2. gate/up : per (selected expert, row tile): the gate and up rows of that
//                expert against every token routed to it (gemv_tile with two
//                matrices), epilogue h = silu(g) * u.
//   3. down    : per (selected expert, row tile): d = Wd h for each of its pairs.
//   4. combine : y[t] = sum_s probs[t][s] * d_(t,s) in slot order.
// Only the selected experts' bytes are read, each once per launch (tokens are
// batched per expert), and nothing is accumulated with atomics.
#include "gemv_core.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

constexpr int kMaxTopK = 32;

// ---------------------------------------------------------------- router ----
// One wave per expert, all tokens.  logits[t][e] = sum_h wr[e][h] x[t][h].
__global__ __launch_bounds__(256) void router_logits_kernel(const float* __restrict__ wr,
                                                            int64_t e, int64_t h,
                                                            const float* __restrict__ x,
                                                            int64_t t, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int64_t ei = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (ei >= e) return;
    const float4* w4 = reinterpret_cast<const float4*>(wr + ei * h);
    const int64_t h4 = h / 4;
    for (int64_t ti = 0; ti < t; ++ti) {
        const float4* x4 = reinterpret_cast<const float4*>(x + ti * h);
        float p[4] = {0.f, 0.f, 0.f, 0.f};
        for (int64_t i = lane; i < h4; i += 64) {
            float4 a = w4[i];
            float4 b = x4[i];
            p[0] += a.x * b.x;
            p[1] += a.y * b.y;
            p[2] += a.z * b.z;
            p[3] += a.w * b.w;
        }
        float s = wave_sum((p[0] + p[1]) + (p[2] + p[3]));
        if (lane == 0) logits[ti * e + ei] = s;
    }
}

// One wave per token: top_k rounds of a wave-wide argmax (ties -> lower index),
// then exp(l - l_max) over the selected logits, normalised in rank order.
__global__ __launch_bounds__(64) void topk_softmax_kernel(const float* __restrict__ logits,
                                                          int64_t e, int top_k,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ probs) {
    const int64_t ti = blockIdx.x;
    const int lane = threadIdx.x;
    const float* l = logits + ti * e;
    constexpr int kPer = 16;  // E <= 1024
    float v[kPer];
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        int64_t i = (int64_t)j * 64 + lane;
        v[j] = i < e ? l[i] : -__builtin_inff();
        if (i >= e) taken |= 1u << j;
    }
    __shared__ int sel[kMaxTopK];
    __shared__ float selv[kMaxTopK];
    for (int s = 0; s < top_k; ++s) {
        float bv = -__builtin_inff();
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            int i = j * 64 + lane;
            bool ok = !(taken >> j & 1u);
            if (ok && (v[j] > bv || (v[j] == bv && i < bi))) {
                bv = v[j];
                bi = i;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            float ov = __shfl_xor(bv, o, 64);
            int oi = __shfl_xor(bi, o, 64);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (bi == 0x7FFFFFFF) bi = 0;  // only non-finite logits left: defined, not meaningful
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == 0) {
            sel[s] = bi;
            selv[s] = bv;
        }
    }
    __syncthreads();
    if (lane == 0) {
        float mx = selv[0];
        float ex[kMaxTopK];
        float z = 0.f;
        for (int s = 0; s < top_k; ++s) {
            ex[s] = expf(selv[s] - mx);
            z += ex[s];
        }
        for (int s = 0; s < top_k; ++s) {
            idx[ti * top_k + s] = sel[s];
            probs[ti * top_k + s] = ex[s] / z;
        }
    }
}

// ---------------------------------------------------------------- layout ----
struct MoeWs {
    int32_t* cnt;     // [E]   pairs per expert
    int32_t* off;     // [E]   first list slot of each expert
    int32_t* active;  // [E]   experts with cnt > 0, ascending
    int32_t* nact;    // [1]
    int32_t* list;    // [P]   pair ids (t*top_k + s) sorted by (expert, pair)
    float* hbuf;      // [P][F]
    float* dbuf;      // [P][H]
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline size_t ints_bytes(int64_t e, int64_t p) { return align256((size_t)(3 * e + 1 + p) * 4); }

MoeWs carve(void* ws, int64_t e, int64_t t, int top_k, int64_t f) {
    const int64_t p = t * top_k;
    uint8_t* base = static_cast<uint8_t*>(ws);
    MoeWs m;
    int32_t* iw = reinterpret_cast<int32_t*>(base);
    m.cnt = iw;
    m.off = iw + e;
    m.active = iw + 2 * e;
    m.nact = iw + 3 * e;
    m.list = iw + 3 * e + 1;
    m.hbuf = reinterpret_cast<float*>(base + ints_bytes(e, p));
    m.dbuf = reinterpret_cast<float*>(base + ints_bytes(e, p) + align256((size_t)p * f * 4));
    return m;
}

// Stable counting sort of the pairs by expert, in one workgroup.
__global__ __launch_bounds__(256) void group_kernel(const int32_t* __restrict__ idx, int64_t p,
                                                    int64_t e, MoeWs ws) {
    extern __shared__ int32_t sh[];
    int32_t* cnt = sh;           // [E]
    int32_t* base = sh + e;      // [E] running placement base
    __shared__ int32_t chunk_e[256];
    const int tid = threadIdx.x;
    for (int64_t i = tid; i < e; i += 256) cnt[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < p; i += 256) {
        int32_t ex = idx[i];
        if (ex < 0 || ex >= e) ex = 0;
        atomicAdd(&cnt[ex], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int32_t run = 0, na = 0;
        for (int64_t i = 0; i < e; ++i) {
            ws.cnt[i] = cnt[i];
            ws.off[i] = run;
            base[i] = run;
            if (cnt[i] > 0) ws.active[na++] = (int32_t)i;
            run += cnt[i];
        }
        for (int64_t i = na; i < e; ++i) ws.active[i] = 0;
        ws.nact[0] = na;
    }
    __syncthreads();
    for (int64_t c0 = 0; c0 < p; c0 += 256) {
        int64_t i = c0 + tid;
        int32_t ex = -1;
        if (i < p) {
            ex = idx[i];
            if (ex < 0 || ex >= e) ex = 0;
        }
        chunk_e[tid] = ex;
        __syncthreads();
        if (i < p) {
            int rank = 0;
            for (int j = 0; j < tid; ++j) rank += chunk_e[j] == ex;
            ws.list[base[ex] + rank] = (int32_t)i;
        }
        __syncthreads();
        if (i < p) atomicAdd(&base[ex], 1);
        __syncthreads();
    }
}

// ------------------------------------------------------- expert GEMVs ----
template <int NB>
struct HEpi {
    float* hbuf;
    int64_t f;
    const int32_t* pairs;  // this group's pair ids
    __device__ void operator()(int b, int64_t r, const float (&v)[2]) const {
        float g = v[0], u = v[1];
        float silu = g / (1.0f + expf(-g));
        hbuf[(int64_t)pairs[b] * f + r] = silu * u;
    }
};

template <int NB>
struct DEpi {
    float* dbuf;
    int64_t h;
    const int32_t* pairs;
    __device__ void operator()(int b, int64_t r, const float (&v)[1]) const {
        dbuf[(int64_t)pairs[b] * h + r] = v[0];
    }
};

template <int FMT, int NB, int ROWS>
__global__ __launch_bounds__(256) void expert_gate_up_kernel(const uint8_t* __restrict__ wg,
                                                             const uint8_t* __restrict__ wu,
                                                             int64_t hdim, int64_t f,
                                                             const float* __restrict__ x,
                                                             int top_k, MoeWs ws) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int a = blockIdx.y;
    if (a >= ws.nact[0]) return;
    const int ex = ws.active[a];
    const int cnt = ws.cnt[ex];
    const int32_t* pairs = ws.list + ws.off[ex];
    const int64_t rb = row_bytes_dev<FMT>(hdim);
    const uint8_t* wm[2] = {wg + (int64_t)ex * f * rb, wu + (int64_t)ex * f * rb};
    for (int g0 = 0; g0 < cnt; g0 += NB) {
        const int batch = min(NB, cnt - g0);
        const float* xr[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            xr[b] = x + (int64_t)(pairs[g0 + (b < batch ? b : 0)] / top_k) * hdim;
        HEpi<NB> epi{ws.hbuf, f, pairs + g0};
        gemv_tile<FMT, NB, ROWS, 2>(lds, wm, f, (int)hdim, rb, xr, batch,
                                    (int64_t)blockIdx.x * ROWS, epi);
        __syncthreads();
    }
}

template <int FMT, int NB, int ROWS>
__global__ __launch_bounds__(256) void expert_down_kernel(const uint8_t* __restrict__ wd,
                                                          int64_t hdim, int64_t f, MoeWs ws) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int a = blockIdx.y;
    if (a >= ws.nact[0]) return;
    const int ex = ws.active[a];
    const int cnt = ws.cnt[ex];
    const int32_t* pairs = ws.list + ws.off[ex];
    const int64_t rb = row_bytes_dev<FMT>(f);
    const uint8_t* wm[1] = {wd + (int64_t)ex * hdim * rb};
    for (int g0 = 0; g0 < cnt; g0 += NB) {
        const int batch = min(NB, cnt - g0);
        const float* xr[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            xr[b] = ws.hbuf + (int64_t)pairs[g0 + (b < batch ? b : 0)] * f;
        DEpi<NB> epi{ws.dbuf, hdim, pairs + g0};
        gemv_tile<FMT, NB, ROWS, 1>(lds, wm, hdim, (int)f, rb, xr, batch,
                                    (int64_t)blockIdx.x * ROWS, epi);
        __syncthreads();
    }
}

// y[t][r] = sum_s probs[t][s] * d[(t*top_k + s)][r], slot order; pairs whose
// expert index is out of range contribute nothing.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ dbuf,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ probs,
                                                      int64_t e, int64_t hdim, int top_k,
                                                      float* __restrict__ y) {
    const int64_t ti = blockIdx.y;
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r >= hdim) return;
    float acc = 0.f;
    for (int s = 0; s < top_k; ++s) {
        int64_t pi = ti * top_k + s;
        int32_t ex = idx[pi];
        float p = (ex >= 0 && ex < e) ? probs[pi] : 0.f;
        acc += p * dbuf[pi * hdim + r];
    }
    y[ti * hdim + r] = acc;
}

template <int FMT, int NB>
hipError_t launch_experts(const uint8_t* wg, const uint8_t* wu, const uint8_t* wd, int64_t e,
                          int64_t hdim, int64_t f, const float* x, int64_t p, int top_k,
                          const MoeWs& ws, hipStream_t s) {
    const unsigned max_act = (unsigned)(p < e ? p : e);
    {
        const int rows = gemv_rows_for(NB, hdim);
        dim3 grid((unsigned)((f + rows - 1) / rows), max_act);
#define GGQ_GU(R)                                                                               \
    hipLaunchKernelGGL((expert_gate_up_kernel<FMT, NB, R>), grid, dim3(256),                    \
                       (GemvCfg<FMT, NB, R, 2>::kLds), s, wg, wu, hdim, f, x, top_k, ws)
        if (rows == 8) GGQ_GU(8);
        else if (rows == 16) GGQ_GU(16);
        else if (rows == 32) GGQ_GU(32);
        else GGQ_GU(64);
#undef GGQ_GU
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    {
        const int rows = gemv_rows_for(NB, f);
        dim3 grid((unsigned)((hdim + rows - 1) / rows), max_act);
#define GGQ_DN(R)                                                                               \
    hipLaunchKernelGGL((expert_down_kernel<FMT, NB, R>), grid, dim3(256),                       \
                       (GemvCfg<FMT, NB, R, 1>::kLds), s, wd, hdim, f, ws)
        if (rows == 8) GGQ_DN(8);
        else if (rows == 16) GGQ_DN(16);
        else if (rows == 32) GGQ_DN(32);
        else GGQ_DN(64);
#undef GGQ_DN
        return hipGetLastError();
    }
}

}  // namespace

hipError_t launch_route(const float* wr, int64_t e, int64_t h, const float* x, int64_t t,
                        int top_k, int32_t* idx, float* probs, float* logits, hipStream_t s) {
    hipLaunchKernelGGL(router_logits_kernel, dim3((unsigned)((e + 3) / 4)), dim3(256), 0, s, wr, e,
                       h, x, t, logits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(topk_softmax_kernel, dim3((unsigned)t), dim3(64), 0, s, logits, e, top_k,
                       idx, probs);
    return hipGetLastError();
}

size_t moe_ws_h_offset(int64_t e, int64_t t, int top_k) { return ints_bytes(e, t * top_k); }

size_t moe_ws_bytes(int64_t e, int64_t t, int top_k, int64_t h, int64_t f) {
    const int64_t p = t * top_k;
    return ints_bytes(e, p) + align256((size_t)p * f * 4) + align256((size_t)p * h * 4);
}

hipError_t launch_moe(int type, const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
                      int64_t e, int64_t h, int64_t f, const float* x, int64_t t,
                      const int32_t* idx, const float* probs, int top_k, float* y, void* ws,
                      hipStream_t s) {
    const int64_t p = t * top_k;
    MoeWs m = carve(ws, e, t, top_k, f);
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(256), (size_t)(2 * e) * 4, s, idx, p, e, m);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // Tokens per expert never exceed T; batch them four at a time.
    if (type == kQ4_K) {
        if (t <= 1) err = launch_experts<kQ4_K, 1>(wg, wu, wd, e, h, f, x, p, top_k, m, s);
        else err = launch_experts<kQ4_K, 4>(wg, wu, wd, e, h, f, x, p, top_k, m, s);
    } else {
        if (t <= 1) err = launch_experts<kQ8_0, 1>(wg, wu, wd, e, h, f, x, p, top_k, m, s);
        else err = launch_experts<kQ8_0, 4>(wg, wu, wd, e, h, f, x, p, top_k, m, s);
    }
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((h + 255) / 256), (unsigned)t), dim3(256), 0,
                       s, m.dbuf, idx, probs, e, h, top_k, y);
    return hipGetLastError();
}

}  // namespace ggq
