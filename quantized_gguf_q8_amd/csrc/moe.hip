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
//   1. group   : a stable counting sort of the T*top_k (token, slot) pairs by
//                expert, giving per-expert pair lists and the ascending list of
//                experts that received any pair.  Up to 256 pairs (decode
//                batches) every workgroup of the next two stages redoes it in
//                LDS, which is cheaper than a launch; beyond that one workgroup
//                writes the lists to the workspace first.
//   2. gate/up : per (selected expert, row tile): the same rows of that expert's
//                gate and up matrices against every token routed to it,
//                epilogue h = silu(g) * u (matrix cores from two tokens on).
//   3. down    : per (selected expert, row tile): d = Wd h for each of its pairs.
//   4. combine : y[t] = sum_s probs[t][s] * d_(t,s) in slot order.
// For one token, 3 and 4 are one kernel (per row tile of H: every slot's down
// product, then the weighted sum in slot order).
// Only the selected experts' bytes are read, once per group of up to 16 tokens
// routed to the expert, and nothing is accumulated with atomics.
#include <algorithm>

#include "gemv_mfma_core.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

constexpr int kMaxTopK = 32;

// ---------------------------------------------------------------- router ----
// One wave per expert, all tokens.  logits[t][e] = sum_h wr[e][h] x[t][h].
// Each 16-byte piece of the router row is loaded once and applied to up to 4
// tokens (token groups spread over the grid's second dimension); per token a
// lane keeps four component sums, combined pairwise, and the wave's lanes are
// summed by a fixed butterfly.
// One token's logit of expert ei by one wave: lane sums over the row pieces
// lane, lane + 64, ... in order (eight requested at a time; a piece index past
// the row re-reads the last piece and is not added), then a fixed butterfly.
__device__ __forceinline__ float router_dot1(const float* __restrict__ wr, int64_t h,
                                             const float* __restrict__ x, int64_t ei, int lane) {
    const float4* w4 = reinterpret_cast<const float4*>(wr + ei * h);
    const float4* x4 = reinterpret_cast<const float4*>(x);
    const int64_t h4 = h / 4;
    constexpr int kU = 8;
    float p[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i0 = lane; i0 < h4; i0 += 64 * kU) {
        float4 a[kU], b[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = min(i0 + 64 * u, h4 - 1);
            a[u] = w4[i];
            b[u] = x4[i];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (i0 + 64 * u < h4) {
                p[0] += a[u].x * b[u].x;
                p[1] += a[u].y * b[u].y;
                p[2] += a[u].z * b[u].z;
                p[3] += a[u].w * b[u].w;
            }
        }
    }
    return wave_sum((p[0] + p[1]) + (p[2] + p[3]));
}

// One workgroup's share: experts 4*bx .. 4*bx+3 (one per wave), token groups
// by, by + gy, ... of kTok tokens.
template <int kTok>
__device__ __forceinline__ void router_logits_block(const float* __restrict__ wr, int64_t e,
                                                    int64_t h, const float* __restrict__ x,
                                                    int64_t t, float* __restrict__ logits, int bx,
                                                    int by, int gy) {
    const int lane = threadIdx.x & 63;
    const int64_t ei = (int64_t)bx * 4 + (threadIdx.x >> 6);
    if (ei >= e) return;
    if constexpr (kTok == 1) {
        const float sum = router_dot1(wr, h, x, ei, lane);
        if (lane == 0) logits[ei] = sum;
        return;
    }
    const float4* w4 = reinterpret_cast<const float4*>(wr + ei * h);
    const int64_t h4 = h / 4;
    // token groups of kTok are spread over by (and looped beyond that)
    for (int64_t t0 = (int64_t)by * kTok; t0 < t; t0 += (int64_t)gy * kTok) {
        const int nt = (int)(t - t0 < kTok ? t - t0 : kTok);
        float p[kTok][4];
#pragma unroll
        for (int j = 0; j < kTok; ++j) p[j][0] = p[j][1] = p[j][2] = p[j][3] = 0.f;
        // pieces lane, lane + 64, ... in order; kU of them requested at a time
        // (a piece index past the row re-reads the last piece and is not added)
        constexpr int kU = 4;
        for (int64_t i0 = lane; i0 < h4; i0 += 64 * kU) {
            float4 a[kU], b[kU][kTok];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t i = min(i0 + 64 * u, h4 - 1);
                a[u] = w4[i];
#pragma unroll
                for (int j = 0; j < kTok; ++j)
                    if (j < nt) b[u][j] = reinterpret_cast<const float4*>(x + (t0 + j) * h)[i];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (i0 + 64 * u < h4) {
#pragma unroll
                    for (int j = 0; j < kTok; ++j) {
                        if (j < nt) {
                            p[j][0] += a[u].x * b[u][j].x;
                            p[j][1] += a[u].y * b[u][j].y;
                            p[j][2] += a[u].z * b[u][j].z;
                            p[j][3] += a[u].w * b[u][j].w;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kTok; ++j) {
            if (j < nt) {
                const float sum = wave_sum((p[j][0] + p[j][1]) + (p[j][2] + p[j][3]));
                if (lane == 0) logits[(t0 + j) * e + ei] = sum;
            }
        }
    }
}

template <int kTok>
__global__ __launch_bounds__(256) void router_logits_kernel(const float* __restrict__ wr,
                                                            int64_t e, int64_t h,
                                                            const float* __restrict__ x,
                                                            int64_t t, float* __restrict__ logits) {
    router_logits_block<kTok>(wr, e, h, x, t, logits, blockIdx.x, blockIdx.y, gridDim.y);
}

// Decode batches: the router and the split of the tokens into fragments for
// the matrix-core expert stages in one launch, on separate workgroups (both
// read only x): workgroups below rgx*rgy compute logits as
// router_logits_kernel<4> does, the rest run xfrag_kernel's workgroups.
template <int FMT>
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr, int64_t e,
                                                           int64_t h, const float* __restrict__ x,
                                                           int64_t t, float* __restrict__ logits,
                                                           int rgx, int rgy, const MJobs jobs, int mt,
                                                           int nslices) {
    const int b = (int)blockIdx.x;
    if (b < rgx * rgy) {
        router_logits_block<4>(wr, e, h, x, t, logits, b % rgx, b / rgx, rgy);
        return;
    }
    const int q = b - rgx * rgy;
    xfrag_block<FMT>(jobs, (int)t, mt, q % (mt * 8), q / (mt * 8), nslices);
}

// Prompt batches: a tile of 16 tokens x 8 experts per workgroup of 128
// threads, thread (token tid/8, expert tid%8), so that a 512-token batch gives
// two workgroups per compute unit.  Columns are staged through LDS 512 at a
// time (the next chunk's rows fetched into registers while the current one is
// used), so each token row and router row is read once per tile instead of
// once per (expert, token group); chunks are long because each one costs a
// memory round trip that only its own compute can hide.  Each thread keeps four component sums over
// 64 columns and adds them to its total every 64 columns (error within about
// 24 rounding units of sum |w x|).
constexpr int kRTT = 16;    // tokens per tile
constexpr int kRTE = 8;     // experts per tile
constexpr int kRKC = 512;   // columns per staged chunk
constexpr int kRRow = kRKC + 4;   // LDS row stride in floats

__global__ __launch_bounds__(128) void router_tile_kernel(const float* __restrict__ wr, int64_t e,
                                                          int64_t h, const float* __restrict__ x,
                                                          int64_t t, float* __restrict__ logits) {
    __shared__ __align__(16) float xs[kRTT * kRRow];
    __shared__ __align__(16) float ws[kRTE * kRRow];
    const int tid = threadIdx.x;
    const int tt = tid / kRTE, te = tid % kRTE;
    const int64_t e0 = (int64_t)blockIdx.x * kRTE;
    // staging: thread loads float4 c = tid (of the chunk's 128) of every row,
    // as buffer loads over the tile's rows: rows past t or e and columns past h
    // read zeros without a select on the loaded value
    const int sc = tid;
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(wr + e0 * h, (uint32_t)((e - e0 < kRTE ? e - e0 : kRTE) * h * 4));
    // token tiles blockIdx.y, + gridDim.y, ... (the grid's y extent is capped)
    for (int64_t t0 = (int64_t)blockIdx.y * kRTT; t0 < t; t0 += (int64_t)gridDim.y * kRTT) {
        const __amdgpu_buffer_rsrc_t rx =
            make_rsrc(x + t0 * h, (uint32_t)((t - t0 < kRTT ? t - t0 : kRTT) * h * 4));
        float4 xv[kRTT], wv[kRTE];
        auto fetch = [&](int64_t k0) {
            const int64_t k = k0 + 4 * sc;
#pragma unroll
            for (int i = 0; i < kRTT; ++i)
                xv[i] = __builtin_bit_cast(float4, buf_load16<false>(
                    rx, k < h ? (uint32_t)((i * h + k) * 4) : kOob));
#pragma unroll
            for (int i = 0; i < kRTE; ++i)
                wv[i] = __builtin_bit_cast(float4, buf_load16<false>(
                    rw, k < h ? (uint32_t)((i * h + k) * 4) : kOob));
        };
        float total = 0.f;
        fetch(0);
        for (int64_t k0 = 0; k0 < h; k0 += kRKC) {
#pragma unroll
            for (int i = 0; i < kRTT; ++i)
                *reinterpret_cast<float4*>(xs + i * kRRow + 4 * sc) = xv[i];
#pragma unroll
            for (int i = 0; i < kRTE; ++i)
                *reinterpret_cast<float4*>(ws + i * kRRow + 4 * sc) = wv[i];
            __syncthreads();
            fetch(k0 + kRKC);   // past h: reads nothing
            const float* xr = xs + tt * kRRow;
            const float* wrow = ws + te * kRRow;
#pragma unroll
            for (int q = 0; q < kRKC / 64; ++q) {
                float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const float4 a = *reinterpret_cast<const float4*>(xr + 64 * q + 4 * c);
                    const float4 b = *reinterpret_cast<const float4*>(wrow + 64 * q + 4 * c);
                    p[0] += a.x * b.x;
                    p[1] += a.y * b.y;
                    p[2] += a.z * b.z;
                    p[3] += a.w * b.w;
                }
                total += (p[0] + p[1]) + (p[2] + p[3]);
            }
            __syncthreads();
        }
        if (t0 + tt < t && e0 + te < e) logits[(t0 + tt) * e + e0 + te] = total;
    }
}

// One wave per token.  The top_k logits (ties -> lower index) are found by a
// radix select over order-preserving 32-bit keys: 32 rounds, each counting
// with wave ballots how many keys lie above a candidate threshold, so no
// round waits on a cross-lane shuffle.  The selected entries are then ranked
// against each other, and exp(l - l_max) over them is normalised in rank
// order.  kPer logits per lane: E <= 64*kPer.
__device__ __forceinline__ uint32_t order_key(float v) {
    if (v != v) return 0u;                  // NaN: below every number
    if (v == 0.f) v = 0.f;                  // -0 and +0 are the same logit
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int ballot_count(bool c) {
    return __builtin_popcountll(__ballot(c));
}

// Top-k of one token's E logits (read through `load(i)`) by one wave: the
// experts in rank order go to sel[0 .. top_k) and their renormalised
// probabilities to selp[], both in LDS.  The wave reads back only its own LDS
// writes (LDS operations of a wave complete in issue order, so only the
// compiler must keep the reads after the writes).
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int kPer, typename Load>
__device__ __forceinline__ void topk_wave(Load load, int64_t e, int top_k, int lane, int* sel,
                                          float* selp) {
    float v[kPer];
    uint32_t key[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t i = (int64_t)j * 64 + lane;
        v[j] = i < e ? load(i) : -__builtin_inff();
        key[j] = i < e ? order_key(v[j]) : 0u;   // padding ranks below every logit
    }
    // threshold = the top_k-th largest key on the bits in `mask`; `want` = how
    // many entries equal to it there are taken (the lowest indices among them).
    // Bits are fixed from the top; once the entries that share the threshold's
    // prefix are exactly the `want` still to take, the selection is settled and
    // the lower bits are left out of the mask.
    uint32_t thr = 0, mask = 0;
    int want = top_k;
    int group = kPer * 64;   // entries whose key matches thr on the mask
    for (int bit = 31; bit >= 0 && group != want; --bit) {
        const uint32_t cand = thr | (1u << bit);
        const uint32_t m = mask | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) cnt += ballot_count((key[j] & m) == cand);
        if (cnt >= want) {
            thr = cand;
            group = cnt;
        } else {
            want -= cnt;
            group -= cnt;
        }
        mask = m;
    }
    // compact the selected entries (index order) into LDS
    __shared__ int cidx[kMaxTopK];
    __shared__ uint32_t ckey[kMaxTopK];
    __shared__ float cval[kMaxTopK];
    __shared__ float selv[kMaxTopK];
    int base = 0, eq_before = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const uint32_t km = key[j] & mask;
        const uint64_t eqm = __ballot(km == thr);
        const uint64_t below = (1ull << lane) - 1ull;   // lanes under this one
        const bool tie_ok = km == thr && eq_before + __builtin_popcountll(eqm & below) < want;
        const bool take = km > thr || tie_ok;
        const uint64_t tm = __ballot(take);
        if (take) {
            const int pos = base + __builtin_popcountll(tm & below);
            cidx[pos] = j * 64 + lane;
            ckey[pos] = key[j];
            cval[pos] = v[j];
        }
        base += __builtin_popcountll(tm);
        eq_before += __builtin_popcountll(eqm);
    }
    wave_lds_order();
    // rank of entry `lane` among the selected: entries with a larger key, or an
    // equal key and a lower index, come first (each selected entry broadcast
    // from its lane)
    const uint32_t mk = lane < top_k ? ckey[lane] : 0u;
    const int mi = lane < top_k ? cidx[lane] : 0;
    const float mv = lane < top_k ? cval[lane] : 0.f;
    int rank = 0;
    for (int q = 0; q < top_k; ++q) {
        const uint32_t kq = (uint32_t)__builtin_amdgcn_readlane((int)mk, q);
        const int iq = __builtin_amdgcn_readlane(mi, q);
        rank += (kq > mk || (kq == mk && iq < mi)) ? 1 : 0;
    }
    if (lane < top_k) {
        sel[rank] = mi;
        selv[rank] = mv;
    }
    wave_lds_order();
    // softmax of the selected logits in rank order: lane s takes exp(v_s - v_0),
    // and the normaliser adds them in rank order
    const float ex = expf((lane < top_k ? selv[lane] : selv[0]) - selv[0]);
    float z = 0.f;
    for (int q = 0; q < top_k; ++q)
        z += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), q));
    if (lane < top_k) selp[lane] = ex / z;
    wave_lds_order();
}

template <int kPer>
__global__ __launch_bounds__(64) void topk_softmax_kernel(const float* __restrict__ logits,
                                                          int64_t e, int top_k,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ probs) {
    __shared__ int sel[kMaxTopK];
    __shared__ float selp[kMaxTopK];
    const int64_t ti = blockIdx.x;
    const int lane = threadIdx.x;
    const float* l = logits + ti * e;
    topk_wave<kPer>([&](int64_t i) { return l[i]; }, e, top_k, lane, sel, selp);
    if (lane < top_k) {
        idx[ti * top_k + lane] = sel[lane];
        probs[ti * top_k + lane] = selp[lane];
    }
}

// One token: the router and the selection in one launch.  Each wave computes
// one expert's logit as router_logits_kernel does and stores it with a
// device-coherent store; the workgroups count themselves on a counter in the
// caller's control block, and the last one to finish runs the selection of
// topk_softmax_kernel on the stored logits and returns the counter to zero.
// The same results as the two kernels, bit for bit.
template <int kPer>
__global__ __launch_bounds__(256) void route1_kernel(const float* __restrict__ wr, int64_t e,
                                                     int64_t h, const float* __restrict__ x,
                                                     int top_k, float* __restrict__ logits,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ probs, uint32_t* ctr) {
    __shared__ int sel[kMaxTopK];
    __shared__ float selp[kMaxTopK];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t ei = (int64_t)blockIdx.x * 4 + (tid >> 6);
    if (ei < e) {
        const float sum = router_dot1(wr, h, x, ei, lane);
        if (lane == 0) __hip_atomic_store(logits + ei, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's logit is stored
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 gridDim.x - 1;
    __syncthreads();
    if (!s_last || tid >= 64) return;
    topk_wave<kPer>([&](int64_t i) {
        return __hip_atomic_load(logits + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }, e, top_k, lane, sel, selp);
    if (lane < top_k) {
        idx[lane] = sel[lane];
        probs[lane] = selp[lane];
    }
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    uint8_t* xfx;     // matrix-core path: fragments of x (xf_layout(Q4_K, H, T/8))
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline size_t ints_bytes(int64_t e, int64_t p) { return align256((size_t)(3 * e + 1 + p) * 4); }

// Fragment regions are sized with the Q4_K layout, which is the larger one.
inline size_t xfx_bytes(int64_t t, int64_t h) { return (size_t)xf_layout(kQ4_K, h, (int)((t + 7) / 8)).bytes; }

MoeWs carve(void* ws, int64_t e, int64_t t, int top_k, int64_t h, int64_t f) {
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
    m.xfx = reinterpret_cast<uint8_t*>(m.dbuf) + align256((size_t)p * h * 4);
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
// Both expert stages are persistent streaming GEMVs over a device-side work
// list (the active experts are known only after routing).  A tile is ROWS rows
// of one selected expert (of both its gate and up matrices in stage 1); a unit
// is one K chunk of a tile for one group of up to NB of the expert's tokens.  A
// workgroup takes tiles blockIdx.x, +gridDim.x, ... and walks each tile's units
// in order; while it computes one unit from LDS, the 16-byte loads of the next
// (weight rows, coalesced, and the gathered activation chunk) are in flight.
// The thread layout and the per-thread decode are those of the decode GEMV:
// thread (row rl, slice s) owns 64 weights of its row per chunk, decodes them
// once and applies them to every token of the group; a row's slices sit in one
// wave and are combined by a fixed butterfly.
template <int FMT, int NB, int ROWS, int NMAT>
struct MoeCfg {
    using Base = GemvCfg<FMT, NB, ROWS, NMAT>;
    static constexpr int SL = Base::SL;
    static constexpr int KC = Base::KC;
    static constexpr int CRB = Base::CRB;
    static constexpr int WRS = Base::WRS;
    static constexpr int XSS = Base::XSS;
    static constexpr int XBS = Base::XBS;
    static constexpr int PPR = CRB / 16;               // 16-byte pieces per row chunk
    static constexpr int MPIECES = ROWS * PPR;          // per matrix
    static constexpr int WPIECES = NMAT * MPIECES;
    static constexpr int WP = (WPIECES + 255) / 256;
    static constexpr int XPIECES = NB * KC / 4;
    static constexpr int XP = (XPIECES + 255) / 256;
    static constexpr int kWBytes = NMAT * ROWS * WRS;
    static constexpr int kXBytes = NB * XBS * 4;
    static constexpr int kSumBytes = FMT == kQ4_K ? NB * SL * 2 * 4 : 0;
    static constexpr int kXBuf = kXBytes + kSumBytes;
    static constexpr int kLds = 2 * kWBytes + 2 * kXBuf;
    // a wave's 64 consecutive weight pieces come from one matrix
    static_assert(MPIECES % 64 == 0, "matrix pieces must be whole waves");
};

struct MoeStage {
    const uint8_t* w[2];   // expert-stacked matrices [E][n][rb] (stage 1: gate, up)
    int64_t n, rb;         // rows per expert matrix, bytes per row
    int32_t k;             // weights per row
    int32_t nchunk;        // K chunks per row
    int32_t tiles;         // row tiles per expert
    const float* x;        // activation rows, ldx floats apart
    int64_t xrows, ldx;
    int32_t xdiv;          // activation row of pair p: p / xdiv
    float* y;              // output row of pair p: y + p * ldy
    int64_t ldy;
    MoeWs ws;              // global lists (written by group_kernel) ...
    const int32_t* idx;    // ... or, with inline_group, rebuilt in LDS from idx (null:
                           // every pair to expert 0, the dense gated FFN)
    int32_t p, e;          // pairs, experts
    int32_t inline_group;
    // One token, gate/up with inline grouping: when set, every workgroup selects
    // the experts itself from the router's logits (idx is not read), and
    // workgroup 0 stores the selection and its probabilities.
    const float* logits;
    int32_t* idx_out;
    float* probs_out;
};

// Pair lists by expert: counts, list offsets, ascending active experts, and the
// pair ids sorted by (expert, pair).  In LDS or in the workspace.
struct MoeLists {
    const int32_t* cnt;
    const int32_t* off;
    const int32_t* active;
    const int32_t* list;
    const int32_t* xrow;   // activation row of each list entry (LDS lists only)
    int nact;
};

constexpr int kInlinePairs = 256;   // up to this many pairs are grouped in LDS

// Element i of a pair list that lives in LDS (LDSL) or in the workspace.  The
// address space is fixed at compile time: read through a generic pointer, an
// LDS list entry is a flat load, which the hardware counts with the global
// loads, so waiting for it would also wait for every weight load issued before.
template <bool LDSL>
__device__ __forceinline__ int32_t lget(const int32_t* p, int i) {
    if constexpr (LDSL) return ((const __attribute__((address_space(3))) int32_t*)p)[i];
    else return ((const __attribute__((address_space(1))) int32_t*)p)[i];
}

__host__ __device__ inline int inline_group_bytes(int64_t e, int64_t p) {
    return (int)((3 * e + 1 + 3 * p) * 4);
}

// Stable counting sort of the p pairs by expert in LDS, by one workgroup of 256
// threads; the same lists group_kernel writes to the workspace.
__device__ __forceinline__ MoeLists group_in_lds(const int32_t* __restrict__ idx, int p, int e,
                                                 int xdiv, int32_t* g) {
    int32_t* cnt = g;
    int32_t* off = g + e;
    int32_t* act = g + 2 * e;
    int32_t* nact = g + 3 * e;
    int32_t* list = g + 3 * e + 1;
    int32_t* ix = list + p;
    int32_t* xr = ix + p;
    const int tid = threadIdx.x;
    if (p <= 64) {
        // One wave, one pair per lane, everything in registers: each lane
        // compares its expert with every pair's (broadcast by readlane) to get
        // its place in the (expert, pair) order, its expert's count and first
        // slot, and the rank of its expert among the distinct ones.  Counts and
        // offsets are written for active experts only, the only ones read.
        if (tid < 64) {
            const int lane = tid;
            int ex = 0x7FFFFFFF;
            if (lane < p) {
                const int32_t v = idx ? idx[lane] : 0;
                ex = (v < 0 || v >= e) ? 0 : v;
            }
            int less = 0, same_before = 0, same = 0;
            for (int j = 0; j < p; ++j) {
                const int exj = __builtin_amdgcn_readlane(ex, j);
                less += exj < ex;
                same_before += (exj == ex) & (j < lane);
                same += exj == ex;
            }
            const bool first = lane < p && same_before == 0;
            const uint64_t fm = __ballot(first);
            int arank = 0;
            for (int j = 0; j < p; ++j) {
                const int exj = __builtin_amdgcn_readlane(ex, j);
                arank += ((fm >> j) & 1ull) && exj < ex;
            }
            if (lane < p) {
                const int pos = less + same_before;
                list[pos] = lane;
                xr[pos] = lane / xdiv;
                if (first) {
                    act[arank] = ex;
                    cnt[ex] = same;
                    off[ex] = less;
                }
            }
            if (lane == 0) nact[0] = __builtin_popcountll(fm);
        }
        __syncthreads();
        return MoeLists{cnt, off, act, list, xr, nact[0]};
    }
    for (int i = tid; i < e; i += 256) cnt[i] = 0;
    for (int i = tid; i < p; i += 256) {
        int32_t ex = idx ? idx[i] : 0;
        ix[i] = (ex < 0 || ex >= e) ? 0 : ex;
    }
    __syncthreads();
    for (int i = tid; i < p; i += 256) atomicAdd(&cnt[ix[i]], 1);
    __syncthreads();
    if (tid < 64) {
        // lane l owns experts [l*per, l*per + per): exclusive scans of the pair
        // counts and of the active flags across the wave
        const int lane = tid;
        const int per = (e + 63) / 64;
        const int b0 = lane * per;
        int sp = 0, sa = 0;
        for (int i = b0; i < min(b0 + per, e); ++i) {
            sp += cnt[i];
            sa += cnt[i] > 0;
        }
        int ip = sp, ia = sa;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int tp = __shfl_up(ip, d, 64);
            const int ta = __shfl_up(ia, d, 64);
            if (lane >= d) {
                ip += tp;
                ia += ta;
            }
        }
        int run = ip - sp, na = ia - sa;
        for (int i = b0; i < min(b0 + per, e); ++i) {
            off[i] = run;
            if (cnt[i] > 0) act[na++] = i;
            run += cnt[i];
        }
        if (lane == 63) nact[0] = ia;
    }
    __syncthreads();
    for (int i = tid; i < p; i += 256) {
        const int ex = ix[i];
        int rank = 0;
        for (int j = 0; j < i; ++j) rank += ix[j] == ex;
        list[off[ex] + rank] = i;
        xr[off[ex] + rank] = i / xdiv;
    }
    __syncthreads();
    return MoeLists{cnt, off, act, list, xr, nact[0]};
}

struct MoeUnit {
    int tile;
    int e;
    int64_t r0;
    int g0;      // first token of the group within the expert's list
    int cnt;     // tokens routed to the expert
    int chunk;
    const int32_t* pairs;
    const int32_t* xrows;  // activation row per pair, or null: pair / xdiv
};

template <int ROWS, bool LDSL>
__device__ __forceinline__ bool moe_locate(const MoeStage& st, const MoeLists& L, int tile,
                                           int total, MoeUnit& u) {
    if (tile >= total) return false;
    u.tile = tile;
    u.e = lget<LDSL>(L.active, tile / st.tiles);
    u.r0 = (int64_t)(tile % st.tiles) * ROWS;
    u.g0 = 0;
    u.cnt = lget<LDSL>(L.cnt, u.e);
    u.chunk = 0;
    const int off = lget<LDSL>(L.off, u.e);
    u.pairs = L.list + off;
    u.xrows = L.xrow ? L.xrow + off : nullptr;
    return true;
}

template <int NB, int ROWS, bool LDSL>
__device__ __forceinline__ bool moe_next(const MoeStage& st, const MoeLists& L, const MoeUnit& p,
                                         int total, MoeUnit& q) {
    q = p;
    if (p.chunk + 1 < st.nchunk) {
        q.chunk = p.chunk + 1;
        return true;
    }
    if (p.g0 + NB < p.cnt) {
        q.g0 = p.g0 + NB;
        q.chunk = 0;
        return true;
    }
    return moe_locate<ROWS, LDSL>(st, L, p.tile + (int)gridDim.x, total, q);
}

template <int FMT, int NB, int ROWS, int NMAT>
struct MoePrefetch {
    using C = MoeCfg<FMT, NB, ROWS, NMAT>;
    uint4 w[C::WP];
    uint4 x[C::XP];

    // Every load is issued whether or not the unit is `live`; when it is not
    // (no next unit) they read past their descriptors and touch no memory (a
    // branch around them would make the compiler wait for them at the join).
    __device__ __forceinline__ void load_w(const MoeStage& st, const MoeUnit& u, int tid,
                                           int wave, bool live) {
        const uint32_t bytes = (uint32_t)(st.n * st.rb);
        const __amdgpu_buffer_rsrc_t r0 =
            make_rsrc_uniform(st.w[0] + (int64_t)u.e * st.n * st.rb, bytes);
        const __amdgpu_buffer_rsrc_t r1 =
            make_rsrc_uniform(st.w[NMAT - 1] + (int64_t)u.e * st.n * st.rb, bytes);
        const uint32_t cb0 = (uint32_t)u.chunk * C::CRB;
        const uint32_t rb = (uint32_t)st.rb;
#pragma unroll
        for (int i = 0; i < C::WP; ++i) {
            const int q = tid + 256 * i;
            const int m = (64 * wave + 256 * i) / C::MPIECES;   // uniform per wave
            const int qm = q - m * C::MPIECES;
            const uint32_t row = (uint32_t)u.r0 + (uint32_t)(qm / C::PPR);
            const uint32_t off = (uint32_t)(qm % C::PPR) * 16;
            const bool ok = live && q < C::WPIECES && row < (uint32_t)st.n && cb0 + off < rb;
            w[i] = buf_load16<true>(m ? r1 : r0, ok ? row * rb + cb0 + off : kOob);
        }
    }

    template <bool LDSL>
    __device__ __forceinline__ void load_x(const MoeStage& st, const MoeUnit& u, int tid,
                                           bool live) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(st.x, (uint32_t)(st.xrows * st.ldx * 4));
        const int k0 = u.chunk * C::KC;
        const int batch = min(NB, u.cnt - u.g0);
#pragma unroll
        for (int i = 0; i < C::XP; ++i) {
            const int q = tid + 256 * i;
            const int b = q / (C::KC / 4);
            const int pos = (q % (C::KC / 4)) * 4;
            uint32_t off = kOob;
            if (live && b < batch && q < C::XPIECES && k0 + pos < st.k) {
                const int64_t xr = u.xrows ? lget<LDSL>(u.xrows, u.g0 + b)
                                           : lget<LDSL>(u.pairs, u.g0 + b) / st.xdiv;
                off = (uint32_t)((xr * st.ldx + k0 + pos) * 4);
            }
            x[i] = buf_load16<false>(r, off);
        }
    }

    __device__ __forceinline__ void store_w(uint8_t* lw, int tid) const {
#pragma unroll
        for (int i = 0; i < C::WP; ++i) {
            const int q = tid + 256 * i;
            if (q < C::WPIECES) {
                const int pr = q / C::PPR;   // row within the NMAT*ROWS stacked tile
                const int off = (q % C::PPR) * 16;
                *reinterpret_cast<uint4*>(lw + pr * C::WRS + off) = w[i];
            }
        }
    }

    __device__ __forceinline__ void store_x(uint8_t* xbuf, int tid, int batch) const {
        float* lx = reinterpret_cast<float*>(xbuf);
        float* lsum = reinterpret_cast<float*>(xbuf + C::kXBytes);
#pragma unroll
        for (int i = 0; i < C::XP; ++i) {
            const int q = tid + 256 * i;
            const int b = q / (C::KC / 4);
            // whole waves only (KC/4 is a multiple of 64); rows past the group's
            // tokens are never read
            if ((C::XPIECES % 256 == 0 || q < C::XPIECES) && b < batch) {
                const int pos = (q % (C::KC / 4)) * 4;
                const float4 v = __builtin_bit_cast(float4, x[i]);
                *reinterpret_cast<float4*>(lx + b * C::XBS + (pos >> 6) * C::XSS + (pos & 63)) = v;
                if constexpr (FMT == kQ4_K) {
                    float t = (v.x + v.y) + (v.z + v.w);
                    t += __shfl_xor(t, 1, 64);
                    t += __shfl_xor(t, 2, 64);
                    t += __shfl_xor(t, 4, 64);
                    if ((q & 7) == 0) lsum[(b * C::SL + (pos >> 6)) * 2 + ((pos >> 5) & 1)] = t;
                }
            }
        }
    }
};

template <int FMT, int NB, int ROWS, int NMAT, bool LDSL>
__device__ __forceinline__ void moe_compute(const MoeStage& st, const MoeUnit& u,
                                            const uint8_t* lw, const uint8_t* xbuf, int s, int rl,
                                            float (&acc)[NMAT][NB]) {
    using C = MoeCfg<FMT, NB, ROWS, NMAT>;
    constexpr int SL = C::SL;
    const float* lx = reinterpret_cast<const float*>(xbuf);
    const float* lsum = reinterpret_cast<const float*>(xbuf + C::kXBytes);
    const int k0 = u.chunk * C::KC;
    const int batch = min(NB, u.cnt - u.g0);
    if (u.r0 + rl < st.n && k0 + s * 64 < st.k) {
        // one 32-weight half at a time: fewer live registers, more resident waves
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                float f[32];
                float sa, mb;
                decode_half<FMT>(lw + (m * ROWS + rl) * C::WRS, s, hf, f, sa, mb);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < batch) {
                        const float4* xv = reinterpret_cast<const float4*>(
                            lx + b * C::XBS + s * C::XSS + 32 * hf);
                        float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const float4 a = xv[i];
                            p[i & 3] += f[4 * i] * a.x + f[4 * i + 1] * a.y + f[4 * i + 2] * a.z +
                                        f[4 * i + 3] * a.w;
                        }
                        float t = sa * ((p[0] + p[1]) + (p[2] + p[3]));
                        if constexpr (FMT == kQ4_K) t -= mb * lsum[(b * SL + s) * 2 + hf];
                        acc[m][b] += t;
                    }
                }
            }
        }
    }
    if (u.chunk == st.nchunk - 1) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int o = 1; o < SL; o <<= 1) acc[m][b] += __shfl_xor(acc[m][b], o, 64);
        if (s == 0 && u.r0 + rl < st.n) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b < batch) {
                    float v = acc[0][b];
                    if constexpr (NMAT == 2) {   // h = silu(gate) * up
                        const float g = acc[0][b];
                        v = g / (1.0f + expf(-g)) * acc[1][b];
                    }
                    st.y[(int64_t)lget<LDSL>(u.pairs, u.g0 + b) * st.ldy + u.r0 + rl] = v;
                }
            }
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[m][b] = 0.f;
    }
}

// SINGLE: launched so that every workgroup computes one unit; LDS then holds
// one W and one x buffer instead of two of each (pair lists follow them).
template <int FMT, int NB, int ROWS, int NMAT, bool SINGLE, bool LDSL>
__global__ __launch_bounds__(256) void moe_stream_kernel(const MoeStage st) {
    using C = MoeCfg<FMT, NB, ROWS, NMAT>;
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t* lw0 = lds;
    uint8_t* lx0 = lds + (SINGLE ? 1 : 2) * C::kWBytes;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = tid % C::SL;
    const int rl = tid / C::SL;
    MoeLists L;
    if constexpr (LDSL) {
        uint8_t* lists = SINGLE ? lds + C::kWBytes + C::kXBuf : lds + C::kLds;
        const int32_t* ix = st.idx;
        if constexpr (NB == 1 && NMAT == 2) {
            if (st.logits) {
                // topk_softmax_kernel's selection, in every workgroup: the
                // logits are 4 bytes per expert, and this saves the launch
                // that would hand the selection over
                __shared__ int s_sel[kMaxTopK];
                __shared__ float s_selp[kMaxTopK];
                if (tid < 64) {
                    auto ld = [&](int64_t i) { return st.logits[i]; };
                    if (st.e <= 128) topk_wave<2>(ld, st.e, st.p, tid, s_sel, s_selp);
                    else topk_wave<4>(ld, st.e, st.p, tid, s_sel, s_selp);
                    if (blockIdx.x == 0 && tid < st.p) {
                        st.idx_out[tid] = s_sel[tid];
                        st.probs_out[tid] = s_selp[tid];
                    }
                }
                __syncthreads();
                ix = s_sel;
            }
        }
        L = group_in_lds(ix, st.p, st.e, st.xdiv, reinterpret_cast<int32_t*>(lists));
    } else {
        L = MoeLists{st.ws.cnt, st.ws.off, st.ws.active, st.ws.list, nullptr, st.ws.nact[0]};
    }
    const int total = L.nact * st.tiles;

    MoeUnit cur;
    if (!moe_locate<ROWS, LDSL>(st, L, blockIdx.x, total, cur)) return;
    MoePrefetch<FMT, NB, ROWS, NMAT> pf;
    pf.load_w(st, cur, tid, wave, true);
    pf.template load_x<LDSL>(st, cur, tid, true);
    pf.store_w(lw0, tid);
    pf.store_x(lx0, tid, min(NB, cur.cnt - cur.g0));
    __syncthreads();

    float acc[NMAT][NB];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[m][b] = 0.f;

    int buf = 0;
    for (;;) {
        MoeUnit nxt;
        const bool more = moe_next<NB, ROWS, LDSL>(st, L, cur, total, nxt);
        if constexpr (SINGLE) {
            // normally one unit per workgroup: nothing to prefetch
            if (more) {
                pf.load_w(st, nxt, tid, wave, true);
                pf.template load_x<LDSL>(st, nxt, tid, true);
            }
        } else {
            // unconditional (past the last unit they read nothing): a branch
            // around the loads would make the compiler wait for them where the
            // paths join, before this unit's compute
            pf.load_w(st, more ? nxt : cur, tid, wave, more);
            pf.template load_x<LDSL>(st, more ? nxt : cur, tid, more);
        }
        moe_compute<FMT, NB, ROWS, NMAT, LDSL>(st, cur, lw0 + buf * C::kWBytes,
                                               lx0 + buf * C::kXBuf, s, rl, acc);
        if (!more) break;
        // With one buffer (more units than planned, e.g. an expert repeated in a
        // token's slots) wait until every wave is done with it.
        if constexpr (SINGLE) __syncthreads();
        else buf ^= 1;
        pf.store_w(lw0 + buf * C::kWBytes, tid);
        pf.store_x(lx0 + buf * C::kXBuf, tid, min(NB, nxt.cnt - nxt.g0));
        __syncthreads();
        cur = nxt;
    }
}

// ------------------------------------------------- matrix-core stage ----
// For two or more tokens the gate/up stage runs on the matrix cores, like the
// batched decode GEMV (with 1-3 tokens per expert the fp32 decode-and-FMA path
// is bound by the vector units there): the tokens are split once per call into
// exact fp16 hi/lo fragments by xfrag_kernel; a unit is one K chunk of 64
// B-operand rows of one selected expert (NMAT = 2: 32 rows of each matrix,
// waves 0-1 gate and 2-3 up; NMAT = 1: 64 rows of one matrix) for one group of
// up to 8 of its tokens, whose fragment rows are gathered lane by lane from the
// per-call fragments.  Weights are staged with 16-byte loads one unit ahead, as
// in the other streaming kernels.
struct MoeMfma {
    const uint8_t* w[2];   // expert-stacked matrices [E][n][rb]
    int64_t n, rb;         // rows per expert matrix, bytes per row
    int32_t k, nchunk, tiles;
    const uint8_t* xf;     // fragments of the activation rows
    int32_t xmt;           // 8-row tiles in xf
    int32_t xdiv;          // activation row of pair p: p / xdiv
    float* y;              // output row of pair p: y + p * ldy
    int64_t ldy;
    MoeWs ws;
    const int32_t* idx;    // null: every pair to expert 0
    int32_t p, e, inline_group;
};

template <int FMT, int NMAT>
struct MoeMCfg {
    // 64 rows, fragments of 8 slots; Q4_K in 256-weight chunks, which fit three
    // workgroups on a compute unit (measured 3% faster at 16 tokens)
    using C = MCfg<FMT, 1, 4, 256>;
    static constexpr int RPM = 64 / NMAT;                 // rows of each matrix per tile
    static constexpr int PPR = C::CRB / 16;                // 16-byte pieces per row chunk
    static constexpr int WMP = RPM * PPR;                  // weight pieces per matrix ...
    static constexpr int WMPAD = (WMP + 63) / 64 * 64;     // ... padded to whole waves
    static constexpr int WPIECES = NMAT * WMPAD;
    static constexpr int WP = (WPIECES + 255) / 256;
    static constexpr int FPIECES = C::kFrag / 16;          // 16-byte fragment pieces
    static constexpr int FP = (FPIECES + 255) / 256;
    static constexpr int MPIECES = C::kMins / 8;           // 8-byte min-term pieces
    static constexpr int MP = (MPIECES + 255) / 256;
    static constexpr int kInvOff = C::kW + C::kFrag + C::kMins;
    static constexpr int kBuf = kInvOff + 32;              // + 2^-S of the 8 slots
    static constexpr int kRed = NMAT == 2 ? 2 * 64 * 2 * 4 : 0;
    static constexpr int kLds = 2 * kBuf + kRed;
};

template <int FMT, int NMAT>
struct MoeMPrefetch {
    using M = MoeMCfg<FMT, NMAT>;
    using C = typename M::C;
    uint4 w[M::WP];
    uint4 f[M::FP];
    uint2 mn[M::MP > 0 ? M::MP : 1];
    float inv;
    int ibatch;     // slots of the unit (inv beyond them is stored as 1)

    uint32_t wok;   // bit i: weight piece i lies inside the matrix (else stored as zeros)

    // A select on a loaded value (zeroing a piece, a default) would wait for
    // the load at once, so out-of-range pieces are zeroed when stored.
    template <bool LDSL>
    __device__ __forceinline__ void load(const MoeMfma& st, const MoeUnit& u, int tid) {
        const int batch = min(8, u.cnt - u.g0);
        const uint32_t cb0 = (uint32_t)u.chunk * C::CRB;
        // weights: piece q of matrix m = q / WMPAD, row q % WMPAD / PPR of the
        // tile; per-lane addresses, clamped to a valid byte
        wok = 0;
#pragma unroll
        for (int i = 0; i < M::WP; ++i) {
            const int q = tid + 256 * i;
            const int m = q / M::WMPAD;
            const int qm = q - m * M::WMPAD;
            const int64_t r = u.r0 + qm / M::PPR;
            const uint32_t off = (uint32_t)(qm % M::PPR) * 16;
            const bool ok = m < NMAT && qm < M::WMP && r < st.n && cb0 + off < st.rb;
            // a select between the two (scalar) matrix pointers: indexing the
            // argument array with a per-lane index would load the pointer from
            // memory, and every weight address would wait for it
            const uint8_t* mat = m == 1 ? st.w[NMAT - 1] : st.w[0];
            const uint8_t* src = mat + ((int64_t)u.e * st.n + (ok ? r : 0)) * st.rb + (ok ? cb0 + off : 0);
            w[i] = load_once16(src);
            wok |= (uint32_t)ok << i;
        }
        // activation fragments gathered per slot: lane l of block b holds slot
        // (l % 16) / 2, hi/lo l % 2, k-octet l / 16
        const XfLayout L = xf_layout(FMT, st.k, st.xmt);
        const __amdgpu_buffer_rsrc_t rf = make_rsrc(st.xf, (uint32_t)L.bytes);
        const int nblk = st.k / 32, nsb = st.k / 256;
#pragma unroll
        for (int i = 0; i < M::FP; ++i) {
            const int q = tid + 256 * i;
            const int blk = q / 64, l = q % 64;
            const int sl = (l & 15) >> 1;
            uint32_t off = kOob;
            const int kb = u.chunk * C::NBLK + blk;
            if (q < M::FPIECES && sl < batch && kb < nblk) {
                const int row = u.xrows ? lget<LDSL>(u.xrows, u.g0 + sl) : lget<LDSL>(u.pairs, u.g0 + sl) / st.xdiv;
                const int sln = 2 * (row & 7) + (l & 1) + 16 * (l >> 4);
                off = (uint32_t)(L.frag + (((int64_t)(row >> 3) * nblk + kb) * 64 + sln) * 16);
            }
            f[i] = buf_load16<false>(rf, off);
        }
        if constexpr (FMT == kQ4_K) {
#pragma unroll
            for (int i = 0; i < M::MP; ++i) {
                const int q = tid + 256 * i;
                const int sb = q / 64, l = q % 64;
                const int sl = (l & 15) >> 1;
                const int ksb = u.chunk * C::NSB + sb;
                uint32_t off = kOob;
                if (q < M::MPIECES && sl < batch && (l >> 4) < 2 && ksb < nsb) {
                    const int row = u.xrows ? lget<LDSL>(u.xrows, u.g0 + sl) : lget<LDSL>(u.pairs, u.g0 + sl) / st.xdiv;
                    const int sln = 2 * (row & 7) + (l & 1) + 16 * (l >> 4);
                    off = (uint32_t)(L.mins + (((int64_t)(row >> 3) * nsb + ksb) * 64 + sln) * 8);
                }
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rf, off, 0, 0);
                mn[i] = make_uint2(v.x, v.y);
            }
        }
        // 2^-S of each slot; slots past the group read slot 0's row and are
        // set to 1 when stored
        ibatch = batch;
        if (tid < 8) {
            const int t = tid < batch ? tid : 0;
            const int row = u.xrows ? lget<LDSL>(u.xrows, u.g0 + t) : lget<LDSL>(u.pairs, u.g0 + t) / st.xdiv;
            inv = __builtin_bit_cast(float,
                                     __builtin_amdgcn_raw_buffer_load_b32(rf, (uint32_t)(L.inv + 4 * row), 0, 0));
        }
    }

    __device__ __forceinline__ void store(uint8_t* buf, int tid) const {
#pragma unroll
        for (int i = 0; i < M::WP; ++i) {
            const int q = tid + 256 * i;
            const int m = q / M::WMPAD, qm = q % M::WMPAD;
            if (m < NMAT && qm < M::WMP)
                *reinterpret_cast<uint4*>(buf + (m * M::RPM + qm / M::PPR) * C::RS +
                                          (qm % M::PPR) * 16) =
                    (wok >> i) & 1u ? w[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < M::FP; ++i) {
            const int q = tid + 256 * i;
            if (q < M::FPIECES) *reinterpret_cast<uint4*>(buf + C::kW + q * 16) = f[i];
        }
        if constexpr (FMT == kQ4_K) {
#pragma unroll
            for (int i = 0; i < M::MP; ++i) {
                const int q = tid + 256 * i;
                if (q < M::MPIECES) *reinterpret_cast<uint2*>(buf + C::kW + C::kFrag + q * 8) = mn[i];
            }
        }
        if (tid < 8) reinterpret_cast<float*>(buf + M::kInvOff)[tid] = tid < ibatch ? inv : 1.f;
    }
};

template <int FMT, int NMAT, bool LDSL>
__global__ __launch_bounds__(256) void moe_mfma_kernel(const MoeMfma st) {
    using M = MoeMCfg<FMT, NMAT>;
    using C = typename M::C;
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;   // B column = row 16 * wave + j of the tile
    const int h = lane >> 4;   // D rows 4h .. 4h+3 = slots 2h, 2h+1 (hi, lo)

    MoeLists L;
    if constexpr (LDSL) {
        L = group_in_lds(st.idx, st.p, st.e, st.xdiv, reinterpret_cast<int32_t*>(lds + M::kLds));
    } else {
        L = MoeLists{st.ws.cnt, st.ws.off, st.ws.active, st.ws.list, nullptr, st.ws.nact[0]};
    }
    const int total = L.nact * st.tiles;

    MoeStage ms{};   // unit walk shared with the streaming kernels
    ms.nchunk = st.nchunk;
    ms.tiles = st.tiles;
    MoeUnit cur;
    if (!moe_locate<M::RPM, LDSL>(ms, L, blockIdx.x, total, cur)) return;
    MoeMPrefetch<FMT, NMAT> pf;
    pf.template load<LDSL>(st, cur, tid);
    pf.store(lds, tid);
    __syncthreads();

    f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    int buf = 0;
    for (;;) {
        MoeUnit nxt;
        const bool more = moe_next<8, M::RPM, LDSL>(ms, L, cur, total, nxt);
        // unconditional (the last unit reloads itself, from L2, unused): a
        // branch around the loads would make the compiler wait for them where
        // the paths join, before this unit's compute
        pf.template load<LDSL>(st, more ? nxt : cur, tid);
        const uint8_t* base = lds + buf * M::kBuf;
        mfma_chunk<FMT, 1, 4, 256>(base, cur.chunk * C::KC, st.k, lane, wave, 0, j, h, acc);
        if (cur.chunk == st.nchunk - 1) {
            const float* invb = reinterpret_cast<const float*>(base + M::kInvOff);
            const int batch = min(8, cur.cnt - cur.g0);
            const int br = 16 * wave + j;
            const int64_t r = cur.r0 + br % M::RPM;
            const float v0 = (acc[0][0] + acc[0][1]) * invb[2 * h];
            const float v1 = (acc[0][2] + acc[0][3]) * invb[2 * h + 1];
            if constexpr (NMAT == 2) {
                // up rows (waves 2, 3) hand their values to the gate rows (waves 0, 1)
                float* red = reinterpret_cast<float*>(lds + 2 * M::kBuf);
                if (wave >= 2) {
                    red[((wave - 2) * 64 + lane) * 2] = v0;
                    red[((wave - 2) * 64 + lane) * 2 + 1] = v1;
                }
                __syncthreads();
                if (wave < 2 && r < st.n) {
                    const float u0 = red[(wave * 64 + lane) * 2], u1 = red[(wave * 64 + lane) * 2 + 1];
                    if (2 * h < batch)
                        st.y[(int64_t)lget<LDSL>(cur.pairs, cur.g0 + 2 * h) * st.ldy + r] = v0 / (1.0f + expf(-v0)) * u0;
                    if (2 * h + 1 < batch)
                        st.y[(int64_t)lget<LDSL>(cur.pairs, cur.g0 + 2 * h + 1) * st.ldy + r] = v1 / (1.0f + expf(-v1)) * u1;
                }
                __syncthreads();
            } else {
                if (r < st.n) {
                    if (2 * h < batch) st.y[(int64_t)lget<LDSL>(cur.pairs, cur.g0 + 2 * h) * st.ldy + r] = v0;
                    if (2 * h + 1 < batch) st.y[(int64_t)lget<LDSL>(cur.pairs, cur.g0 + 2 * h + 1) * st.ldy + r] = v1;
                }
            }
            acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (!more) break;
        buf ^= 1;
        pf.store(lds + buf * M::kBuf, tid);
        __syncthreads();
        cur = nxt;
    }
}

// Q4_K gate/up weights streamed line by line.  A row of K = 2048 weights is
// eight 144-byte super-blocks in nine 128-byte lines, and super-block c lies
// in lines c and c + 1 (lines 9 (c / 8) + c % 8 and the next for longer rows),
// so after the first super-block of each eight a row needs one new line per
// chunk.  Whole 144-byte chunks read with streaming loads fetched the line two
// chunks share twice (1.56x the algorithmic bytes at 16 tokens); here every
// line is read once.  The lines of a row sit in a three-slot ring in LDS, slot
// = the workgroup's running line count mod 3: the next chunk's new line goes
// to the slot the current chunk does not read, and when the next chunk needs
// two new lines the second is stored after a further barrier, once the
// current chunk's first line is no longer read.  Used when K is a multiple of
// 2048 and the matrices start on 128-byte boundaries (every row then does too).
template <int NMAT>
struct MoeRingCfg {
    // the piece map below covers 32 rows of each of two matrices
    static_assert(NMAT == 2, "gate and up");
    using C = MCfg<kQ4_K, 1, 4, 256>;
    static constexpr int RPM = 64 / NMAT;
    // 100 dwords per row: the 16 rows a wave reads start on distinct
    // multiples of 4 banks
    static constexpr int RS = 3 * 128 + 16;
    static constexpr int kRing = 64 * RS;
    // min-term operands of lane groups 0, 1 only (groups 2, 3 are zero)
    static constexpr int kMins = 32 * 8;
    static constexpr int kInvOff = C::kFrag + kMins;
    static constexpr int kXBuf = kInvOff + 32;
    // one activation buffer (the next chunk's fragments are stored after a
    // barrier), and the up-to-gate hand-off at a tile's end in its own area:
    // with two activation buffers only three workgroups shared a compute unit
    static constexpr int kRed = 2 * 64 * 2 * 4;
    static constexpr int kLds = kRing + kXBuf + kRed;
    static constexpr int FPIECES = C::kFrag / 16;
    static constexpr int FP = (FPIECES + 255) / 256;
    static constexpr int MPIECES = kMins / 8;
    static constexpr int MP = (MPIECES + 255) / 256;
};

template <int NMAT>
struct MoeRingPrefetch {
    using R = MoeRingCfg<NMAT>;
    using C = typename R::C;
    uint4 w[4];         // 64 rows x up to two lines x 8 pieces = 1024 pieces
    uint4 f[R::FP];
    uint2 mn[R::MP];
    float inv;
    int ibatch;
    uint32_t wst;       // bit i: piece i is stored
    uint32_t wzero;     // bit i: ... as zeros (row past the matrix)
    uint32_t wlate;     // bit i: ... after the current chunk's reads (second of two new lines)
    uint32_t wdst[4];   // ring byte offset of piece i

    // g: ring position of the unit's first line of this chunk.
    template <bool LDSL>
    __device__ __forceinline__ void load(const MoeMfma& st, const MoeUnit& u, int g, int tid) {
        const int cp = u.chunk & 7;
        const bool two = cp == 0;   // first chunk of eight: both of its lines are new
        const uint32_t l0 = 9u * (uint32_t)(u.chunk >> 3) + (uint32_t)cp;
        const uint32_t bytes = (uint32_t)(st.n * st.rb);
        const __amdgpu_buffer_rsrc_t r0 =
            make_rsrc_uniform(st.w[0] + (int64_t)u.e * st.n * st.rb, bytes);
        const __amdgpu_buffer_rsrc_t r1 =
            make_rsrc_uniform(st.w[NMAT - 1] + (int64_t)u.e * st.n * st.rb, bytes);
        const uint32_t rb = (uint32_t)st.rb;
        wst = 0;
        wzero = 0;
        wlate = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i;
            // two lines: q = (matrix, row, line, piece); one line: (matrix, row,
            // piece) and pieces 2, 3 idle.  The matrix is uniform per i.
            const int m = two ? i >> 1 : i;
            const int r = two ? (q & 511) >> 4 : (q & 255) >> 3;
            const int line = two ? (q >> 3) & 1 : 1;
            const int byte = (q & 7) * 16;
            const bool live = m < NMAT;
            const uint32_t row = (uint32_t)u.r0 + (uint32_t)r;
            const bool in = live && row < (uint32_t)st.n;
            w[i] = buf_load16<true>(m == 1 ? r1 : r0, in ? row * rb + (l0 + line) * 128 + byte : kOob);
            wst |= (uint32_t)live << i;
            wzero |= (uint32_t)(live && !in) << i;
            wlate |= (uint32_t)(live && two && line == 1) << i;
            wdst[i] = (uint32_t)((m * R::RPM + r) * R::RS + ((g + line) % 3) * 128 + byte);
        }
        const int batch = min(8, u.cnt - u.g0);
        const XfLayout L = xf_layout(kQ4_K, st.k, st.xmt);
        const __amdgpu_buffer_rsrc_t rf = make_rsrc(st.xf, (uint32_t)L.bytes);
        const int nblk = st.k / 32, nsb = st.k / 256;
#pragma unroll
        for (int i = 0; i < R::FP; ++i) {
            const int q = tid + 256 * i;
            const int blk = q / 64, l = q % 64;
            const int sl = (l & 15) >> 1;
            uint32_t off = kOob;
            const int kb = u.chunk * C::NBLK + blk;
            if (q < R::FPIECES && sl < batch && kb < nblk) {
                const int row = u.xrows ? lget<LDSL>(u.xrows, u.g0 + sl) : lget<LDSL>(u.pairs, u.g0 + sl) / st.xdiv;
                const int sln = 2 * (row & 7) + (l & 1) + 16 * (l >> 4);
                off = (uint32_t)(L.frag + (((int64_t)(row >> 3) * nblk + kb) * 64 + sln) * 16);
            }
            f[i] = buf_load16<false>(rf, off);
        }
#pragma unroll
        for (int i = 0; i < R::MP; ++i) {
            const int q = tid + 256 * i;
            const int sb = q / 64, l = q % 64;
            const int sl = (l & 15) >> 1;
            const int ksb = u.chunk + sb;
            uint32_t off = kOob;
            if (q < R::MPIECES && sl < batch && ksb < nsb) {
                const int row = u.xrows ? lget<LDSL>(u.xrows, u.g0 + sl) : lget<LDSL>(u.pairs, u.g0 + sl) / st.xdiv;
                const int sln = 2 * (row & 7) + (l & 1) + 16 * (l >> 4);
                off = (uint32_t)(L.mins + (((int64_t)(row >> 3) * nsb + ksb) * 64 + sln) * 8);
            }
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rf, off, 0, 0);
            mn[i] = make_uint2(v.x, v.y);
        }
        ibatch = batch;
        if (tid < 8) {
            const int t = tid < batch ? tid : 0;
            const int row = u.xrows ? lget<LDSL>(u.xrows, u.g0 + t) : lget<LDSL>(u.pairs, u.g0 + t) / st.xdiv;
            inv = __builtin_bit_cast(float,
                                     __builtin_amdgcn_raw_buffer_load_b32(rf, (uint32_t)(L.inv + 4 * row), 0, 0));
        }
    }

    // Everything but the late pieces (store_late, after a barrier).
    __device__ __forceinline__ void store(uint8_t* ring, uint8_t* xb, int tid) const {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (((wst & ~wlate) >> i) & 1u)
                *reinterpret_cast<uint4*>(ring + wdst[i]) = (wzero >> i) & 1u ? make_uint4(0, 0, 0, 0) : w[i];
#pragma unroll
        for (int i = 0; i < R::FP; ++i) {
            const int q = tid + 256 * i;
            if (q < R::FPIECES) *reinterpret_cast<uint4*>(xb + q * 16) = f[i];
        }
#pragma unroll
        for (int i = 0; i < R::MP; ++i) {
            const int q = tid + 256 * i;
            if (q < R::MPIECES) *reinterpret_cast<uint2*>(xb + C::kFrag + q * 8) = mn[i];
        }
        if (tid < 8) reinterpret_cast<float*>(xb + R::kInvOff)[tid] = tid < ibatch ? inv : 1.f;
    }

    __device__ __forceinline__ void store_late(uint8_t* ring) const {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if ((wlate >> i) & 1u)
                *reinterpret_cast<uint4*>(ring + wdst[i]) = (wzero >> i) & 1u ? make_uint4(0, 0, 0, 0) : w[i];
    }
};

// The products of one super-block (chunk) from the ring: the Q4_K arithmetic
// of mfma_chunk (gemv_mfma_core.h) for one 16-row group, with the bytes read
// from the two ring slots that hold the super-block.
template <int NMAT>
__device__ __forceinline__ void ring_chunk(const uint8_t* ring, const uint8_t* xb, int g, int cp,
                                           int lane, int wave, int j, int h, f32x4& acc) {
    using R = MoeRingCfg<NMAT>;
    using C = typename R::C;
    const uint8_t* rowp = ring + (16 * wave + j) * R::RS;
    const uint8_t* b0 = rowp + (g % 3) * 128;
    const uint8_t* b1 = rowp + ((g + 1) % 3) * 128;
    const int s0 = 16 * cp;   // super-block start inside its first line
    // every LDS read of the chunk first, then the arithmetic
    const uint4 hd = *reinterpret_cast<const uint4*>(b0 + s0);
    uint2 qv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int x = s0 + 16 + 32 * c + 8 * h;   // 8-byte pieces never straddle a line
        qv[c] = *reinterpret_cast<const uint2*>(x < 128 ? b0 + x : b1 + (x - 128));
    }
    f16x8 aop[8];
#pragma unroll
    for (int sub = 0; sub < 8; ++sub)
        aop[sub] = *reinterpret_cast<const f16x8*>(xb + sub * 1024 + lane * 16);
    const f16x4 xop = h < 2 ? *reinterpret_cast<const f16x4*>(xb + C::kFrag + lane * 8)
                            : f16x4{0, 0, 0, 0};
    const float d = half_bits_to_float(hd.x);
    const float dmin = half_bits_to_float(hd.x >> 16);
    const Q4KScales scl = q4k_unpack(hd.y, hd.z, hd.w);
    f32x4 dsb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const int sub = 2 * c + hi;
            uint32_t scj, mj;
            q4k_sub(scl, sub, scj, mj);
            const _Float16 sch = (_Float16)(float)scj;
            const _Float16 msch = (_Float16)(-1024.f * (float)scj);
            const f16x2 sc2 = {sch, sch};
            const f16x2 msc2 = {msch, msch};
            const uint32_t n0 = hi ? (qv[c].x >> 4) & 0x0F0F0F0Fu : qv[c].x & 0x0F0F0F0Fu;
            const uint32_t n1 = hi ? (qv[c].y >> 4) & 0x0F0F0F0Fu : qv[c].y & 0x0F0F0F0Fu;
            uint32_t b4[4];
            q4x4_to_f16(n0, sc2, msc2, b4[0], b4[1]);
            q4x4_to_f16(n1, sc2, msc2, b4[2], b4[3]);
            const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(b4[0], b4[1], b4[2], b4[3]));
            dsb = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[sub], bop, dsb, 0, 0, 0);
        }
    }
    // min term: B[k][col] = m_k of this row for k < 8, zero above
    const uint32_t mv = h == 0 ? scl.mnl : scl.mnh;
    uint32_t m0 = 0, m1 = 0;
    if (h < 2) {
        const uint32_t e = 0x64646464u;
        const f16x2 off = {(_Float16)1024.f, (_Float16)1024.f};
        m0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, mv, 0x04010400u)) - off);
        m1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, mv, 0x04030402u)) - off);
    }
    const f16x4 mop = __builtin_bit_cast(f16x4, make_uint2(m0, m1));
    const f32x4 dmn = __builtin_amdgcn_mfma_f32_16x16x16f16(xop, mop, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    acc += d * dsb - (32.f * dmin) * dmn;
}

// moe_mfma_kernel for Q4_K with the weights in line rings (see MoeRingCfg).
// At most 128 VGPRs, so that four waves share a SIMD as the LDS allows four
// workgroups per compute unit.
template <int NMAT, bool LDSL>
__global__ __launch_bounds__(256, 4) void moe_ring_kernel(const MoeMfma st) {
    using R = MoeRingCfg<NMAT>;
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;
    const int h = lane >> 4;
    uint8_t* ring = lds;
    uint8_t* xbufs = lds + R::kRing;

    MoeLists L;
    if constexpr (LDSL) {
        L = group_in_lds(st.idx, st.p, st.e, st.xdiv, reinterpret_cast<int32_t*>(lds + R::kLds));
    } else {
        L = MoeLists{st.ws.cnt, st.ws.off, st.ws.active, st.ws.list, nullptr, st.ws.nact[0]};
    }
    const int total = L.nact * st.tiles;

    MoeStage ms{};
    ms.nchunk = st.nchunk;
    ms.tiles = st.tiles;
    MoeUnit cur;
    if (!moe_locate<R::RPM, LDSL>(ms, L, blockIdx.x, total, cur)) return;
    int g = 0;   // ring position of the current chunk's first line
    MoeRingPrefetch<NMAT> pf;
    pf.template load<LDSL>(st, cur, g, tid);
    pf.store(ring, xbufs, tid);
    pf.store_late(ring);
    __syncthreads();

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (;;) {
        MoeUnit nxt;
        const bool more = moe_next<8, R::RPM, LDSL>(ms, L, cur, total, nxt);
        const int gn = g + ((nxt.chunk & 7) == 0 ? 2 : 1);
        // unconditional (the last unit reloads itself, never stored)
        pf.template load<LDSL>(st, more ? nxt : cur, more ? gn : g, tid);
        const uint8_t* xb = xbufs;
        ring_chunk<NMAT>(ring, xb, g, cur.chunk & 7, lane, wave, j, h, acc);
        if (cur.chunk == st.nchunk - 1) {
            const float* invb = reinterpret_cast<const float*>(xb + R::kInvOff);
            const int batch = min(8, cur.cnt - cur.g0);
            const int br = 16 * wave + j;
            const int64_t r = cur.r0 + br % R::RPM;
            const float v0 = (acc[0] + acc[1]) * invb[2 * h];
            const float v1 = (acc[2] + acc[3]) * invb[2 * h + 1];
            if constexpr (NMAT == 2) {
                // up rows (waves 2, 3) hand their values to the gate rows (waves 0, 1)
                float* red = reinterpret_cast<float*>(xbufs + R::kXBuf);
                if (wave >= 2) {
                    red[((wave - 2) * 64 + lane) * 2] = v0;
                    red[((wave - 2) * 64 + lane) * 2 + 1] = v1;
                }
                __syncthreads();
                if (wave < 2 && r < st.n) {
                    const float u0 = red[(wave * 64 + lane) * 2], u1 = red[(wave * 64 + lane) * 2 + 1];
                    if (2 * h < batch)
                        st.y[(int64_t)lget<LDSL>(cur.pairs, cur.g0 + 2 * h) * st.ldy + r] = v0 / (1.0f + expf(-v0)) * u0;
                    if (2 * h + 1 < batch)
                        st.y[(int64_t)lget<LDSL>(cur.pairs, cur.g0 + 2 * h + 1) * st.ldy + r] = v1 / (1.0f + expf(-v1)) * u1;
                }
                __syncthreads();
            } else {
                if (r < st.n) {
                    if (2 * h < batch) st.y[(int64_t)lget<LDSL>(cur.pairs, cur.g0 + 2 * h) * st.ldy + r] = v0;
                    if (2 * h + 1 < batch) st.y[(int64_t)lget<LDSL>(cur.pairs, cur.g0 + 2 * h + 1) * st.ldy + r] = v1;
                }
            }
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (!more) break;
        // every wave is done with this chunk's fragments and ring slots: the
        // next chunk's fragments and lines (both of them when it starts a group
        // of eight) can be stored
        __syncthreads();
        pf.store(ring, xbufs, tid);
        if ((nxt.chunk & 7) == 0) pf.store_late(ring);
        __syncthreads();
        cur = nxt;
        g = gn;
    }
}

// y[t][r] = sum_s probs[t][s] * d[(t*top_k + s)][r], slot order.  Pairs whose
// expert index is out of range were grouped with expert 0 and carry whatever
// its matrices gave; their term is skipped (not multiplied by 0), so a
// non-finite expert 0 cannot reach y through them.
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
        if (ex >= 0 && ex < e) acc += probs[pi] * dbuf[pi * hdim + r];
    }
    y[ti * hdim + r] = acc;
}

// ------------------------------------------ one token: down and combine ----
// y = sum over slots s, in slot order, of probs[s] * (Wd[idx[s]] h_s) in one
// launch, for one token (no per-slot rows written, no combine launch).  A
// workgroup owns `rows` rows of H and every unit (slot, row, 64-weight piece
// of F) of them, at most kD1Units per thread, all fetched at once; the h of
// every slot is staged in LDS once.  A unit's partial sum goes to LDS and the
// row's owner adds them up in (slot, piece) order.  Slots whose expert index
// lies outside [0, E) contribute nothing and their weights are not read.
constexpr int kD1Units = 4;
// h of a slot is kept in LDS as 64-float pieces kD1Stride floats apart, so the
// pieces that the lanes of a wave read at once start on different banks
constexpr int kD1Stride = 68;

struct Down1Args {
    const uint8_t* wd;     // [E][H][rb]
    const float* h;        // [top_k][F]
    const int32_t* idx;    // [top_k]
    const float* probs;    // [top_k]
    float* y;              // [H]
    int64_t e, hdim, rb;   // experts, rows of H, bytes per row of Wd
    int32_t f, top_k, rows, upr;   // F, slots, rows per workgroup, pieces per row (F / 64)
};

template <int FMT>
struct D1Raw;
template <>
struct D1Raw<kQ4_K> {
    uint4 hdr, q0, q1;   // super-block header, the piece's 32 quant bytes
};
template <>
struct D1Raw<kQ8_0> {
    uint32_t v[17];      // two blocks, 68 bytes
};

// The loads of a thread's down units (at most U): workgroup rows r0 .. r0 +
// rows - 1, slot experts from ex_of(slot).
template <int FMT, int U, typename ExOf>
__device__ __forceinline__ void d1_load(const Down1Args& a, int64_t r0, int tid, ExOf ex_of,
                                        D1Raw<FMT> (&raw)[U], bool (&live)[U]) {
    const int per_slot = a.rows * a.upr;
    const int total = a.top_k * per_slot;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int u = tid + 256 * j;
        const int slot = u / per_slot, rem = u % per_slot;
        const int64_t row = r0 + rem / a.upr;
        const int piece = rem % a.upr;
        const int ex = u < total ? ex_of(slot) : -1;
        live[j] = u < total && ex >= 0 && ex < a.e && row < a.hdim;
        if (!live[j]) continue;
        const uint8_t* rp = a.wd + ((int64_t)ex * a.hdim + row) * a.rb;
        if constexpr (FMT == kQ4_K) {
            const uint8_t* sb = rp + (int64_t)(piece / 4) * kQ4Bytes;
            raw[j].hdr = load_once16(sb);
            raw[j].q0 = load_once16(sb + 16 + 32 * (piece % 4));
            raw[j].q1 = load_once16(sb + 32 + 32 * (piece % 4));
        } else {
            const uint32_t* q = reinterpret_cast<const uint32_t*>(rp + (int64_t)piece * 2 * kQ8Bytes);
#pragma unroll
            for (int i = 0; i < 17; ++i) raw[j].v[i] = __builtin_nontemporal_load(q + i);
        }
    }
}

// h of every slot into LDS as [top_k][F / 64][kD1Stride] (rows of slots without
// an expert are copied too and never used), 16 bytes per lane, eight loads per
// lane in flight at a time (one at a time, each load is a round trip).
constexpr int kD1HBatch = 8;

__device__ __forceinline__ void d1_stage_h(const Down1Args& a, float* lh, int tid) {
    const int hq = a.top_k * a.f / 4;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(a.h, (uint32_t)hq * 16u);
    for (int i0 = 0; i0 < hq; i0 += 256 * kD1HBatch) {
        u32x4 v[kD1HBatch];
#pragma unroll
        for (int j = 0; j < kD1HBatch; ++j) {
            const int i = i0 + 256 * j + tid;
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, i < hq ? (uint32_t)i * 16u : kOob, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kD1HBatch; ++j) {
            const int i = i0 + 256 * j + tid;
            if (i < hq) {
                const int c = 4 * i, slot = c / a.f, col = c % a.f;
                *reinterpret_cast<u32x4*>(lh + (slot * a.upr + col / 64) * kD1Stride + col % 64) = v[j];
            }
        }
    }
}

// The units' partial sums, then each (slot, row) and each row in order, with
// h staged in lh and the slots' experts and weights in s_ex / s_p (all visible
// to every thread on entry).
template <int FMT, int U>
__device__ __forceinline__ void d1_finish(const Down1Args& a, int64_t r0, int tid,
                                          const D1Raw<FMT> (&raw)[U], const bool (&live)[U],
                                          float* lh, float* lpart, const int* s_ex,
                                          const float* s_p) {
    const int per_slot = a.rows * a.upr;
    const int total = a.top_k * per_slot;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int u = tid + 256 * j;
        if (u >= total) break;
        float part = 0.f;
        if (live[j]) {
            const int slot = u / per_slot;
            const int piece = (u % per_slot) % a.upr;
            const float* hv = lh + (slot * a.upr + piece) * kD1Stride;
            if constexpr (FMT == kQ4_K) {
                // low nibbles: sub-block 2c, weights 64c + l; high: 2c + 1, 64c + 32 + l
                const int c = piece % 4;
                const Q4KScales sc = q4k_unpack(raw[j].hdr.y, raw[j].hdr.z, raw[j].hdr.w);
                uint32_t sc0, m0, sc1, m1;
                q4k_sub(sc, 2 * c, sc0, m0);
                q4k_sub(sc, 2 * c + 1, sc1, m1);
                const float d = half_bits_to_float(raw[j].hdr.x);
                const float dmin = half_bits_to_float(raw[j].hdr.x >> 16);
                const uint32_t qw[8] = {raw[j].q0.x, raw[j].q0.y, raw[j].q0.z, raw[j].q0.w,
                                        raw[j].q1.x, raw[j].q1.y, raw[j].q1.z, raw[j].q1.w};
                float dl = 0.f, dh = 0.f, sl = 0.f, sh = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 xl = reinterpret_cast<const float4*>(hv)[i];
                    const float4 xh = reinterpret_cast<const float4*>(hv + 32)[i];
                    const uint32_t lo = qw[i] & 0x0F0F0F0Fu, hi = (qw[i] >> 4) & 0x0F0F0F0Fu;
                    dl += ubyte_f(lo, 0) * xl.x + ubyte_f(lo, 1) * xl.y + ubyte_f(lo, 2) * xl.z +
                          ubyte_f(lo, 3) * xl.w;
                    dh += ubyte_f(hi, 0) * xh.x + ubyte_f(hi, 1) * xh.y + ubyte_f(hi, 2) * xh.z +
                          ubyte_f(hi, 3) * xh.w;
                    sl += (xl.x + xl.y) + (xl.z + xl.w);
                    sh += (xh.x + xh.y) + (xh.z + xh.w);
                }
                part = d * (float)sc0 * dl - dmin * (float)m0 * sl +
                       (d * (float)sc1 * dh - dmin * (float)m1 * sh);
            } else {
                // block 0: scale bytes 0-1, quants 2-33; block 1: 34-35, 36-67
                const uint32_t* v = raw[j].v;
                float d0 = 0.f, d1 = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 x0 = reinterpret_cast<const float4*>(hv)[i];
                    const float4 x1 = reinterpret_cast<const float4*>(hv + 32)[i];
                    const uint32_t q0 = __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2);
                    const uint32_t q1 = v[9 + i];
                    d0 += sbyte_f(q0, 0) * x0.x + sbyte_f(q0, 1) * x0.y + sbyte_f(q0, 2) * x0.z +
                          sbyte_f(q0, 3) * x0.w;
                    d1 += sbyte_f(q1, 0) * x1.x + sbyte_f(q1, 1) * x1.y + sbyte_f(q1, 2) * x1.z +
                          sbyte_f(q1, 3) * x1.w;
                }
                part = half_bits_to_float(v[0]) * d0 + half_bits_to_float(v[8] >> 16) * d1;
            }
        }
        lpart[u] = part;
    }
    __syncthreads();

    // each (slot, row): its pieces in order, into the h buffer (no longer read);
    // then each row: the slots in order, weighted
    for (int i = tid; i < a.top_k * a.rows; i += 256) {
        const float* pp = lpart + (i / a.rows) * per_slot + (i % a.rows) * a.upr;
        float dsum = 0.f;
        for (int q = 0; q < a.upr; ++q) dsum += pp[q];
        lh[i] = dsum;
    }
    __syncthreads();
    if (tid < a.rows && r0 + tid < a.hdim) {
        float acc = 0.f;
        for (int s = 0; s < a.top_k; ++s) {
            const int ex = s_ex[s];
            if (ex >= 0 && ex < a.e) acc += s_p[s] * lh[s * a.rows + tid];
        }
        a.y[r0 + tid] = acc;
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void moe_down1_kernel(const Down1Args a) {
    extern __shared__ __align__(16) uint8_t lds[];
    float* lh = reinterpret_cast<float*>(lds);   // [top_k][F / 64][kD1Stride]
    float* lpart = lh + a.top_k * a.upr * kD1Stride;   // one partial sum per unit
    __shared__ int s_ex[kMaxTopK];
    __shared__ float s_p[kMaxTopK];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * a.rows;
    // weights of this thread's units (loads first: they take longest)
    D1Raw<FMT> raw[kD1Units];
    bool live[kD1Units];
    d1_load<FMT, kD1Units>(a, r0, tid, [&](int slot) { return a.idx[slot]; }, raw, live);
    d1_stage_h(a, lh, tid);
    if (tid < a.top_k) {
        s_ex[tid] = a.idx[tid];
        s_p[tid] = a.probs[tid];
    }
    __syncthreads();
    d1_finish<FMT, kD1Units>(a, r0, tid, raw, live, lh, lpart, s_ex, s_p);
}

int moe_device_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    return cus;
}

// Resident workgroups per compute unit of a stage kernel at an LDS size (the
// last two sizes asked are cached).
template <int FMT, int NB, int ROWS, int NMAT, bool SINGLE, bool LDSL>
int stage_blocks_per_cu(size_t lds) {
    static size_t key[2] = {0, 0};
    static int val[2] = {0, 0};
    for (int i = 0; i < 2; ++i)
        if (key[i] == lds) return val[i];
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &v, moe_stream_kernel<FMT, NB, ROWS, NMAT, SINGLE, LDSL>, 256, lds) != hipSuccess ||
        v <= 0)
        v = 1;
    key[1] = key[0];
    val[1] = val[0];
    key[0] = lds;
    val[0] = v;
    return v;
}

// `max_group`: the most tokens any expert can receive in this call.  LDSL: the
// pair lists are rebuilt in LDS by every workgroup (st.inline_group).
template <int FMT, int NB, int ROWS, int NMAT, bool LDSL>
hipError_t launch_stage_l(MoeStage st, int64_t slots, int64_t max_group, hipStream_t s) {
    using C = MoeCfg<FMT, NB, ROWS, NMAT>;
    const size_t lists = LDSL ? inline_group_bytes(st.e, st.p) : 0;
    st.nchunk = (st.k + C::KC - 1) / C::KC;
    st.tiles = (int32_t)((st.n + ROWS - 1) / ROWS);
    const int64_t most = slots * st.tiles;
    // One unit per workgroup (a single K chunk, one token group, every tile
    // resident at once): the second LDS buffer would never be used, and
    // leaving it out lets more workgroups share a compute unit.  The kernel
    // stays correct if a workgroup does get more units (it then reuses the one
    // buffer behind a barrier).
    if constexpr (NB == 1) {
        const size_t lds1 = (size_t)C::kWBytes + C::kXBuf + lists;
        const int64_t cap1 =
            (int64_t)stage_blocks_per_cu<FMT, NB, ROWS, NMAT, true, LDSL>(lds1) * moe_device_cus();
        if (st.nchunk == 1 && max_group <= NB && most <= cap1) {
            hipLaunchKernelGGL((moe_stream_kernel<FMT, NB, ROWS, NMAT, true, LDSL>),
                               dim3((unsigned)most), dim3(256), lds1, s, st);
            return hipGetLastError();
        }
    }
    const size_t lds = C::kLds + lists;
    const int per_cu = stage_blocks_per_cu<FMT, NB, ROWS, NMAT, false, LDSL>(lds);
    const int64_t cap = (int64_t)per_cu * moe_device_cus();
    const unsigned grid = (unsigned)(most < cap ? most : cap);
    hipLaunchKernelGGL((moe_stream_kernel<FMT, NB, ROWS, NMAT, false, LDSL>), dim3(grid),
                       dim3(256), lds, s, st);
    return hipGetLastError();
}

template <int FMT, int NB, int ROWS, int NMAT>
hipError_t launch_stage(const MoeStage& st, int64_t slots, int64_t max_group, hipStream_t s) {
    return st.inline_group ? launch_stage_l<FMT, NB, ROWS, NMAT, true>(st, slots, max_group, s)
                           : launch_stage_l<FMT, NB, ROWS, NMAT, false>(st, slots, max_group, s);
}

// Rows per tile.  One token (NB = 1): the most rows whose K chunk covers the
// whole row (8 rows for K <= 2048, 16 for K <= 1024), so a tile is one unit --
// the stages are latency-bound there and a second chunk is a second round
// trip.  Otherwise the largest of 64/32/16 (at least 2*NB) that still gives
// every compute unit two tiles when `slots` experts are active.
template <int FMT, int NB, int NMAT>
hipError_t launch_stage_rows(const MoeStage& st, int64_t slots, int64_t max_group,
                             hipStream_t s) {
    if constexpr (NB == 1) {
        if (st.k <= 64 * (256 / 16)) return launch_stage<FMT, 1, 16, NMAT>(st, slots, max_group, s);
        if (st.k <= 64 * (256 / 8)) return launch_stage<FMT, 1, 8, NMAT>(st, slots, max_group, s);
    }
    const int64_t want = 2 * (int64_t)moe_device_cus();
    int rows = 64;
    while (rows > 16 && rows / 2 >= 2 * NB && slots * ((st.n + rows - 1) / rows) < want) rows /= 2;
    if (rows == 64) return launch_stage<FMT, NB, 64, NMAT>(st, slots, max_group, s);
    if constexpr (2 * NB <= 32)
        if (rows == 32) return launch_stage<FMT, NB, 32, NMAT>(st, slots, max_group, s);
    if constexpr (2 * NB <= 16)
        if (rows == 16) return launch_stage<FMT, NB, 16, NMAT>(st, slots, max_group, s);
    return launch_stage<FMT, NB, 32, NMAT>(st, slots, max_group, s);
}

template <int FMT, int NMAT, bool LDSL>
hipError_t launch_mstage_l(MoeMfma st, int64_t slots, hipStream_t s) {
    using M = MoeMCfg<FMT, NMAT>;
    using C = typename M::C;
    const size_t lds = M::kLds + (LDSL ? inline_group_bytes(st.e, st.p) : 0);
    static size_t per_cu_lds = 0;
    static int per_cu = 0;
    if (per_cu_lds != lds) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(moe_mfma_kernel<FMT, NMAT, LDSL>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, moe_mfma_kernel<FMT, NMAT, LDSL>, 256,
                                                         lds) != hipSuccess ||
            v <= 0)
            v = 1;
        per_cu = v;
        per_cu_lds = lds;
    }
    st.nchunk = (st.k + C::KC - 1) / C::KC;
    st.tiles = (int32_t)((st.n + M::RPM - 1) / M::RPM);
    const int64_t most = slots * st.tiles;
    const int64_t cap = (int64_t)per_cu * moe_device_cus();
    const unsigned grid = (unsigned)(most < cap ? most : cap);
    hipLaunchKernelGGL((moe_mfma_kernel<FMT, NMAT, LDSL>), dim3(grid), dim3(256), lds, s, st);
    return hipGetLastError();
}

template <int NMAT, bool LDSL>
hipError_t launch_ring_l(MoeMfma st, int64_t slots, hipStream_t s) {
    using R = MoeRingCfg<NMAT>;
    const size_t lds = R::kLds + (LDSL ? inline_group_bytes(st.e, st.p) : 0);
    static size_t per_cu_lds = 0;
    static int per_cu = 0;
    if (per_cu_lds != lds) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(moe_ring_kernel<NMAT, LDSL>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, moe_ring_kernel<NMAT, LDSL>, 256, lds) !=
                hipSuccess ||
            v <= 0)
            v = 1;
        per_cu = v;
        per_cu_lds = lds;
    }
    st.nchunk = st.k / 256;
    st.tiles = (int32_t)((st.n + R::RPM - 1) / R::RPM);
    const int64_t most = slots * st.tiles;
    const int64_t cap = (int64_t)per_cu * moe_device_cus();
    const unsigned grid = (unsigned)(most < cap ? most : cap);
    hipLaunchKernelGGL((moe_ring_kernel<NMAT, LDSL>), dim3(grid), dim3(256), lds, s, st);
    return hipGetLastError();
}

template <int FMT, int NMAT>
hipError_t launch_mstage(const MoeMfma& st, int64_t slots, hipStream_t s) {
    const bool ring = FMT == kQ4_K && NMAT == 2 && st.k % 2048 == 0 &&
                      reinterpret_cast<uintptr_t>(st.w[0]) % 128 == 0 &&
                      reinterpret_cast<uintptr_t>(st.w[NMAT - 1]) % 128 == 0;
    if constexpr (NMAT == 2)
        if (ring)
            return st.inline_group ? launch_ring_l<NMAT, true>(st, slots, s)
                                   : launch_ring_l<NMAT, false>(st, slots, s);
    return st.inline_group ? launch_mstage_l<FMT, NMAT, true>(st, slots, s)
                           : launch_mstage_l<FMT, NMAT, false>(st, slots, s);
}

// Split `rows` activation rows of K floats into the fragments at xf.
template <int FMT>
hipError_t launch_split(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* xf,
                        hipStream_t s) {
    MJobs jobs{};
    jobs.count = 1;
    jobs.j[0].x = x;
    jobs.j[0].xf = xf;
    jobs.j[0].ldx = ldx;
    jobs.j[0].k = (int32_t)k;
    const int mt = (int)((rows + 7) / 8);
    const dim3 grid((unsigned)(mt * 8), (unsigned)((k / 32 + kXfragSlice - 1) / kXfragSlice));
    hipLaunchKernelGGL(xfrag_kernel<FMT>, grid, dim3(256), 0, s, jobs, (int)rows, mt);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_experts_mfma(const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
                               int64_t e, int64_t hdim, int64_t f, const float* x, int64_t t,
                               int top_k, const int32_t* idx, const MoeWs& ws, hipStream_t s,
                               bool split_done = false) {
    const int64_t p = t * top_k;
    const int64_t slots = p < e ? p : e;
    const bool inl = p <= kInlinePairs;
    hipError_t err = hipSuccess;
    if (!split_done) {   // else the router launch split x already
        err = launch_split<FMT>(x, t, hdim, hdim, ws.xfx, s);
        if (err != hipSuccess) return err;
    }
    MoeMfma a{};
    a.w[0] = wg;
    a.w[1] = wu;
    a.n = f;
    a.rb = row_bytes(FMT, hdim);
    a.k = (int32_t)hdim;
    a.xf = ws.xfx;
    a.xmt = (int32_t)((t + 7) / 8);
    a.xdiv = top_k;
    a.y = ws.hbuf;
    a.ldy = f;
    a.ws = ws;
    a.idx = idx;
    a.p = (int32_t)p;
    a.e = (int32_t)e;
    a.inline_group = inl;
    err = launch_mstage<FMT, 2>(a, slots, s);
    if (err != hipSuccess) return err;
    // The down stage stays on the vector units: with K = F short, splitting h
    // into fragments costs a launch that the matrix cores do not win back.
    MoeStage d{};
    d.idx = idx;
    d.p = (int32_t)p;
    d.e = (int32_t)e;
    d.inline_group = inl;
    d.w[0] = wd;
    d.w[1] = wd;
    d.n = hdim;
    d.rb = row_bytes(FMT, f);
    d.k = (int32_t)f;
    d.x = ws.hbuf;
    d.xrows = p;
    d.ldx = f;
    d.xdiv = 1;
    d.y = ws.dbuf;
    d.ldy = hdim;
    d.ws = ws;
    return launch_stage_rows<FMT, 4, 1>(d, slots, t, s);
}

// The router's logits of one token, from which the one-token gate/up stage
// selects the experts itself (storing the selection in idx / probs).
struct MoeSelect {
    const float* logits;
    int32_t* idx;
    float* probs;
};

template <int FMT, int NB>
hipError_t launch_experts(const uint8_t* wg, const uint8_t* wu, const uint8_t* wd, int64_t e,
                          int64_t hdim, int64_t f, const float* x, int64_t t, int top_k,
                          const int32_t* idx, const MoeWs& ws, hipStream_t s,
                          bool down = true, const MoeSelect* sel = nullptr) {
    const int64_t p = t * top_k;
    const int64_t slots = p < e ? p : e;
    const bool inl = p <= kInlinePairs;
    MoeStage a{};
    a.idx = idx;
    if (sel) {
        a.logits = sel->logits;
        a.idx_out = sel->idx;
        a.probs_out = sel->probs;
    }
    a.p = (int32_t)p;
    a.e = (int32_t)e;
    a.inline_group = inl;
    a.w[0] = wg;
    a.w[1] = wu;
    a.n = f;
    a.rb = row_bytes(FMT, hdim);
    a.k = (int32_t)hdim;
    a.x = x;
    a.xrows = t;
    a.ldx = hdim;
    a.xdiv = top_k;
    a.y = ws.hbuf;
    a.ldy = f;
    a.ws = ws;
    hipError_t err = launch_stage_rows<FMT, NB, 2>(a, slots, t, s);
    if (err != hipSuccess || !down) return err;
    MoeStage d{};
    d.idx = idx;
    d.p = (int32_t)p;
    d.e = (int32_t)e;
    d.inline_group = inl;
    d.w[0] = wd;
    d.w[1] = wd;
    d.n = hdim;
    d.rb = row_bytes(FMT, f);
    d.k = (int32_t)f;
    d.x = ws.hbuf;
    d.xrows = p;
    d.ldx = f;
    d.xdiv = 1;
    d.y = ws.dbuf;
    d.ldy = hdim;
    d.ws = ws;
    return launch_stage_rows<FMT, NB, 1>(d, slots, t, s);
}

}  // namespace

static hipError_t launch_topk(const float* logits, int64_t e, int64_t t, int top_k, int32_t* idx,
                              float* probs, hipStream_t s) {
    if (e <= 128)
        hipLaunchKernelGGL((topk_softmax_kernel<2>), dim3((unsigned)t), dim3(64), 0, s, logits, e,
                           top_k, idx, probs);
    else if (e <= 256)
        hipLaunchKernelGGL((topk_softmax_kernel<4>), dim3((unsigned)t), dim3(64), 0, s, logits, e,
                           top_k, idx, probs);
    else
        hipLaunchKernelGGL((topk_softmax_kernel<16>), dim3((unsigned)t), dim3(64), 0, s, logits, e,
                           top_k, idx, probs);
    return hipGetLastError();
}

hipError_t launch_route(const float* wr, int64_t e, int64_t h, const float* x, int64_t t,
                        int top_k, int32_t* idx, float* probs, float* logits, hipStream_t s) {
    if (t >= 32) {
        const int64_t tiles = (t + kRTT - 1) / kRTT;
        hipLaunchKernelGGL(router_tile_kernel,
                           dim3((unsigned)((e + kRTE - 1) / kRTE), (unsigned)(tiles < 65535 ? tiles : 65535)),
                           dim3(128), 0, s, wr, e, h, x, t, logits);
    } else {
        const int64_t groups = (t + 3) / 4;
        if (t == 1)
            hipLaunchKernelGGL((router_logits_kernel<1>), dim3((unsigned)((e + 3) / 4), 1), dim3(256), 0,
                               s, wr, e, h, x, t, logits);
        else
            hipLaunchKernelGGL((router_logits_kernel<4>),
                               dim3((unsigned)((e + 3) / 4), (unsigned)(groups < 64 ? groups : 64)),
                               dim3(256), 0, s, wr, e, h, x, t, logits);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_topk(logits, e, t, top_k, idx, probs, s);
}

// The gate and up projections of a dense gated FFN with the SiLU*up epilogue:
// the expert stages with one expert that every token is routed to.
hipError_t launch_swiglu(int type, const uint8_t* wg, const uint8_t* wu, int64_t n, int64_t k,
                         const float* x, int64_t ldx, float* h, int64_t ldh, int batch, void* ws,
                         hipStream_t s) {
    const bool q4 = type == kQ4_K;
    const int64_t rb = row_bytes(type, k);
    if (batch <= 1) {
        MoeStage a{};
        a.idx = nullptr;
        a.p = batch;
        a.e = 1;
        a.inline_group = 1;
        a.w[0] = wg;
        a.w[1] = wu;
        a.n = n;
        a.rb = rb;
        a.k = (int32_t)k;
        a.x = x;
        a.xrows = batch;
        a.ldx = ldx;
        a.xdiv = 1;
        a.y = h;
        a.ldy = ldh;
        return q4 ? launch_stage_rows<kQ4_K, 1, 2>(a, 1, 1, s)
                  : launch_stage_rows<kQ8_0, 1, 2>(a, 1, 1, s);
    }
    uint8_t* xf = static_cast<uint8_t*>(ws);
    hipError_t err = q4 ? launch_split<kQ4_K>(x, batch, k, ldx, xf, s)
                        : launch_split<kQ8_0>(x, batch, k, ldx, xf, s);
    if (err != hipSuccess) return err;
    MoeMfma a{};
    a.w[0] = wg;
    a.w[1] = wu;
    a.n = n;
    a.rb = rb;
    a.k = (int32_t)k;
    a.xf = xf;
    a.xmt = (int32_t)((batch + 7) / 8);
    a.xdiv = 1;
    a.y = h;
    a.ldy = ldh;
    a.idx = nullptr;
    a.p = batch;
    a.e = 1;
    a.inline_group = 1;
    return q4 ? launch_mstage<kQ4_K, 2>(a, 1, s) : launch_mstage<kQ8_0, 2>(a, 1, s);
}

// The one-token down-and-combine kernel takes every (slot, row, piece) unit of
// a workgroup's rows in one pass and keeps the h of all slots in LDS.
static bool down1_fits(int64_t f, int top_k) {
    // dynamic LDS (h of every slot, one partial per unit) plus the kernel's
    // static slot arrays within the default 64 KiB
    return ((int64_t)top_k * (f / 64) * kD1Stride + (int64_t)kD1Units * 256 + 2 * kMaxTopK) * 4 <= 65536 &&
           (int64_t)top_k * (f / 64) <= (int64_t)kD1Units * 256;
}

static hipError_t launch_down1(int type, const uint8_t* wd, int64_t e, int64_t hdim, int64_t f,
                        const float* hbuf, const int32_t* idx, const float* probs, int top_k,
                        float* y, hipStream_t s) {
    Down1Args a;
    a.wd = wd;
    a.h = hbuf;
    a.idx = idx;
    a.probs = probs;
    a.y = y;
    a.e = e;
    a.hdim = hdim;
    a.rb = row_bytes(type, f);
    a.f = (int32_t)f;
    a.top_k = top_k;
    a.upr = (int32_t)(f / 64);
    // as many rows as the unit budget allows, but no more than it takes to
    // give every compute unit two workgroups
    const int64_t cap = (int64_t)kD1Units * 256 / ((int64_t)top_k * a.upr);
    const int64_t wgs = 2 * (int64_t)moe_device_cus();
    const int64_t spread = (hdim + wgs - 1) / wgs;
    a.rows = (int32_t)std::max<int64_t>(1, std::min<int64_t>({cap, spread, 256}));
    const size_t lds = ((size_t)top_k * a.upr * kD1Stride + (size_t)top_k * a.rows * a.upr) * 4;
    const unsigned grid = (unsigned)((hdim + a.rows - 1) / a.rows);
    if (type == kQ4_K)
        hipLaunchKernelGGL(moe_down1_kernel<kQ4_K>, dim3(grid), dim3(256), lds, s, a);
    else
        hipLaunchKernelGGL(moe_down1_kernel<kQ8_0>, dim3(grid), dim3(256), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const float* dbuf, const int32_t* idx, const float* probs, int64_t e,
                          int64_t h, int64_t t, int top_k, float* y, hipStream_t s) {
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((h + 255) / 256), (unsigned)t), dim3(256), 0,
                       s, dbuf, idx, probs, e, h, top_k, y);
    return hipGetLastError();
}

size_t moe_ws_h_offset(int64_t e, int64_t t, int top_k) { return ints_bytes(e, t * top_k); }

size_t moe_ws_bytes(int64_t e, int64_t t, int top_k, int64_t h, int64_t f) {
    const int64_t p = t * top_k;
    return ints_bytes(e, p) + align256((size_t)p * f * 4) + align256((size_t)p * h * 4) +
           align256(xfx_bytes(t, h));
}

// x_split: two or more tokens whose fragments the router launch already wrote.
static hipError_t launch_moe_impl(int type, const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
                                  int64_t e, int64_t h, int64_t f, const float* x, int64_t t,
                                  const int32_t* idx, const float* probs, int top_k, float* y,
                                  void* ws, hipStream_t s, bool x_split) {
    const int64_t p = t * top_k;
    MoeWs m = carve(ws, e, t, top_k, h, f);
    hipError_t err = hipSuccess;
    if (p > kInlinePairs) {
        hipLaunchKernelGGL(group_kernel, dim3(1), dim3(256), (size_t)(2 * e) * 4, s, idx, p, e, m);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // One token: the vector-unit streaming stages.  Two or more: the matrix-core
    // stages (groups of up to 8 of an expert's tokens per pass).
    const bool q4 = type == kQ4_K;
    if (t == 1 && down1_fits(f, top_k)) {
        // one token: gate/up stage, then down and combine in one kernel
        err = q4 ? launch_experts<kQ4_K, 1>(wg, wu, wd, e, h, f, x, t, top_k, idx, m, s, false)
                 : launch_experts<kQ8_0, 1>(wg, wu, wd, e, h, f, x, t, top_k, idx, m, s, false);
        if (err != hipSuccess) return err;
        return launch_down1(type, wd, e, h, f, m.hbuf, idx, probs, top_k, y, s);
    }
    if (t <= 1) err = q4 ? launch_experts<kQ4_K, 1>(wg, wu, wd, e, h, f, x, t, top_k, idx, m, s)
                         : launch_experts<kQ8_0, 1>(wg, wu, wd, e, h, f, x, t, top_k, idx, m, s);
    else err = q4 ? launch_experts_mfma<kQ4_K>(wg, wu, wd, e, h, f, x, t, top_k, idx, m, s, x_split)
                  : launch_experts_mfma<kQ8_0>(wg, wu, wd, e, h, f, x, t, top_k, idx, m, s, x_split);
    if (err != hipSuccess) return err;
    return launch_combine(m.dbuf, idx, probs, e, h, t, top_k, y, s);
}

hipError_t launch_moe(int type, const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
                      int64_t e, int64_t h, int64_t f, const float* x, int64_t t,
                      const int32_t* idx, const float* probs, int top_k, float* y, void* ws,
                      hipStream_t s) {
    return launch_moe_impl(type, wg, wu, wd, e, h, f, x, t, idx, probs, top_k, y, ws, s, false);
}

// The router and the token split in one launch (2..31 tokens), then the top-k.
template <int FMT>
static hipError_t launch_route_split(const float* wr, int64_t e, int64_t h, const float* x, int64_t t,
                                     int top_k, int32_t* idx, float* probs, float* logits,
                                     uint8_t* xf, hipStream_t s) {
    MJobs jobs{};
    jobs.count = 1;
    jobs.j[0].x = x;
    jobs.j[0].xf = xf;
    jobs.j[0].ldx = h;
    jobs.j[0].k = (int32_t)h;
    const int mt = (int)((t + 7) / 8);
    const int nslices = (int)((h / 32 + kXfragSlice - 1) / kXfragSlice);
    const int rgx = (int)((e + 3) / 4), rgy = (int)((t + 3) / 4);
    const unsigned grid = (unsigned)(rgx * rgy + mt * 8 * nslices);
    hipLaunchKernelGGL((router_split_kernel<FMT>), dim3(grid), dim3(256), 0, s, wr, e, h, x, t,
                       logits, rgx, rgy, jobs, mt, nslices);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_topk(logits, e, t, top_k, idx, probs, s);
}

size_t moe_layer_ws_bytes(int64_t e, int64_t t, int top_k, int64_t h, int64_t f) {
    return kCtrlBytes + moe_ws_bytes(e, t, top_k, h, f);
}

hipError_t launch_moe_layer(int type, const float* wr, const uint8_t* wg, const uint8_t* wu,
                            const uint8_t* wd, int64_t e, int64_t h, int64_t f, const float* x,
                            int64_t t, int top_k, float* logits, int32_t* idx, float* probs,
                            float* y, void* ws, hipStream_t s) {
    uint8_t* mws = static_cast<uint8_t*>(ws) + kCtrlBytes;
    hipError_t err = hipSuccess;
    if (t == 1 && e <= 256 && down1_fits(f, top_k)) {
        // router; gate/up, whose workgroups each take the selection from the
        // logits (workgroup 0 stores it); down and the combine
        hipLaunchKernelGGL((router_logits_kernel<1>), dim3((unsigned)((e + 3) / 4), 1), dim3(256), 0,
                           s, wr, e, h, x, t, logits);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        const MoeWs m = carve(mws, e, t, top_k, h, f);
        const MoeSelect sel{logits, idx, probs};
        err = type == kQ4_K
                  ? launch_experts<kQ4_K, 1>(wg, wu, wd, e, h, f, x, t, top_k, idx, m, s, false, &sel)
                  : launch_experts<kQ8_0, 1>(wg, wu, wd, e, h, f, x, t, top_k, idx, m, s, false, &sel);
        if (err != hipSuccess) return err;
        return launch_down1(type, wd, e, h, f, m.hbuf, idx, probs, top_k, y, s);
    }
    if (t == 1) {
        // router and selection in one launch (the counter: word 0 of the control block)
        uint32_t* ctr = static_cast<uint32_t*>(ws);
        const dim3 grid((unsigned)((e + 3) / 4));
        if (e <= 128)
            hipLaunchKernelGGL((route1_kernel<2>), grid, dim3(256), 0, s, wr, e, h, x, top_k, logits,
                               idx, probs, ctr);
        else if (e <= 256)
            hipLaunchKernelGGL((route1_kernel<4>), grid, dim3(256), 0, s, wr, e, h, x, top_k, logits,
                               idx, probs, ctr);
        else
            hipLaunchKernelGGL((route1_kernel<16>), grid, dim3(256), 0, s, wr, e, h, x, top_k,
                               logits, idx, probs, ctr);
        err = hipGetLastError();
    } else if (t < 32) {
        // the router and the split of the tokens into fragments in one launch
        const MoeWs m = carve(mws, e, t, top_k, h, f);
        err = type == kQ4_K
                  ? launch_route_split<kQ4_K>(wr, e, h, x, t, top_k, idx, probs, logits, m.xfx, s)
                  : launch_route_split<kQ8_0>(wr, e, h, x, t, top_k, idx, probs, logits, m.xfx, s);
        if (err != hipSuccess) return err;
        return launch_moe_impl(type, wg, wu, wd, e, h, f, x, t, idx, probs, top_k, y, mws, s, true);
    } else {
        err = launch_route(wr, e, h, x, t, top_k, idx, probs, logits, s);
    }
    if (err != hipSuccess) return err;
    return launch_moe(type, wg, wu, wd, e, h, f, x, t, idx, probs, top_k, y, mws, s);
}

}  // namespace ggq
