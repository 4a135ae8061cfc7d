// gemv_mfma.hip -- batched decode GEMV (batch 2..16) on the matrix cores.
//
// Same product as quant_gemv (Phobos README, "Inference"); the operand
// conversions and the per-chunk MFMA arithmetic are in gemv_mfma_core.h.
//
// Work decomposition: a workgroup (4 waves) owns 16*WM rows; each wave owns 16
// rows (the 16 columns of the B operand) and every WK-th block of each K chunk
// (WM*WK = 4).  Chunks of weights and activation fragments are staged through LDS
// with the same register-prefetch pipeline as the VALU path.  The WK partials of
// a tile are summed in LDS in wave order at the end of its K walk.
//
// Scheduling: workgroups are persistent and take work items (a row tile, or
// one of its K parts) from a counter, largest first.  With whole tiles only, a
// grid of ~3 workgroups per CU drew one or two 64-row tiles each and a quarter
// of the chip idled for the last third of the launch; halves even this out.
// Short, long-K matrices (a few dozen row tiles) are cut into up to 16 K parts
// when the workspace has room for their partial sums.
//
// Weights are read with ordinary (not streaming) loads: a 64-row K chunk
// starts and ends inside 128-byte lines, and the next chunk's loads find the
// shared line in L2 only if it was not marked for early eviction.
#include <algorithm>
#include <climits>
#include <map>
#include <utility>

#include "gemv_mfma_core.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

// A unit's position, with its job's fields copied in: they stay in scalar
// registers, where reading them from the job table on every unit cost a
// scalar-load round trip on the critical path.
struct MPos {
    int job, chunk, cend;   // chunk: current K chunk; cend: one past the item's last
    int64_t r0;
    const uint8_t* w;
    uint8_t* xf;
    float* out;             // where the item's results go: y, or its partial-sum plane
    int64_t n, ostride;     // rows; distance between batch rows of `out`
    uint32_t rb;
    int k, add;             // add: atomic add into a zeroed y (one of two K halves)
};

// Work item -> (job, row tile, K range).  Items of a job are numbered tile by
// tile, halves of a split tile next to each other; the first half takes the
// odd chunk.
template <int RWG>
__device__ __forceinline__ MPos mlocate(const MJobs& jobs, int item) {
    // The item is the same for the whole workgroup (it may come through LDS,
    // where the compiler cannot see that): with it in a scalar register the
    // job fields are scalar loads and the buffer descriptors built from them
    // stay scalar (a per-lane descriptor becomes a loop over lanes).
    item = __builtin_amdgcn_readfirstlane(item);
    int j = 0;
    while (j + 1 < jobs.count && item >= jobs.j[j + 1].item0) ++j;
    const MJob& jb = jobs.j[j];
    const int local = item - jb.item0;
    MPos p;
    p.job = j;
    p.w = jb.w;
    p.xf = jb.xf;
    p.n = jb.n;
    p.rb = (uint32_t)jb.rb;
    p.k = jb.k;
    p.out = jb.y;
    p.ostride = jb.ldy;
    p.add = jb.nsplit == 2;
    if (jb.nsplit > 1) {
        const int part = local % jb.nsplit;
        p.r0 = (int64_t)(local / jb.nsplit) * RWG;
        p.chunk = part * jb.cpp;
        p.cend = min(jb.nchunk, p.chunk + jb.cpp);
        if (jb.nsplit > 2) {
            p.out = jb.part + (int64_t)part * jobs.batch * jb.n;
            p.ostride = jb.n;
        }
    } else {
        p.r0 = (int64_t)local * RWG;
        p.chunk = 0;
        p.cend = jb.nchunk;
    }
    return p;
}

template <int FMT, int MT, int WM>
struct MPrefetch {
    using C = MCfg<FMT, MT, WM>;
    uint4 w[C::WP];
    uint4 f[C::FP];
    // Per-thread piece offsets, set when the job changes, so that a unit's loads
    // cost one add (or none) per piece: the unit's origin goes into the
    // descriptor base instead.
    uint32_t wrel[C::WP];    // weight piece: byte offset from the unit's first byte, kOob if none
    uint32_t woff[C::WP];    // its byte offset inside the row chunk (partial last chunks)
    uint32_t frel[C::FP];    // fragment piece: byte offset in the job region at chunk 0, kOob if none
    uint32_t fpos[C::FP];    // Q4_K: position of its block in the chunk, in bytes of its kind
    int job;

    __device__ __forceinline__ void set_job(const MPos& jb, int tid) {
        const uint32_t rb = jb.rb;
#pragma unroll
        for (int i = 0; i < C::WP; ++i) {
            const int q = tid + 256 * i;
            const uint32_t pr = (uint32_t)q / (C::CRB / 16);
            woff[i] = ((uint32_t)q % (C::CRB / 16)) * 16;
            wrel[i] = q < C::WPIECES ? pr * rb + woff[i] : kOob;
        }
        const XfLayout L = xf_layout(FMT, jb.k, MT);
        const int nblk = jb.k / 32;
        const int nsb = jb.k / 256;
#pragma unroll
        for (int i = 0; i < C::FP; ++i) {
            const int q = tid + 256 * i;
            const int o = q * 16;  // byte offset inside a chunk's fragment staging
            frel[i] = kOob;
            fpos[i] = 0;
            if (q < C::FPIECES) {
                if (o < C::kFrag) {
                    const int t = o / (C::NBLK * 1024);
                    const int rem = o % (C::NBLK * 1024);
                    frel[i] = (uint32_t)(L.frag + (int64_t)t * nblk * 1024 + rem);
                    fpos[i] = (uint32_t)(rem & ~1023);
                } else if constexpr (FMT == kQ4_K) {
                    const int o2 = o - C::kFrag;
                    const int t = o2 / (C::NSB * 512);
                    const int rem = o2 % (C::NSB * 512);
                    frel[i] = (uint32_t)(L.mins + (int64_t)t * nsb * 512 + rem);
                    fpos[i] = (uint32_t)(rem & ~511);
                }
            }
        }
    }

    // Out-of-range pieces (rows past N, bytes past a row, blocks past K) load
    // from an offset beyond the descriptor and come back as zeros.
    __device__ __forceinline__ void load(const MJobs& jobs, const MPos& p, int tid) {
        const MPos& jb = p;
        if (p.job != job) {
            set_job(p, tid);
            job = p.job;
        }
        const uint32_t rb = p.rb;
        const uint32_t cb0 = (uint32_t)p.chunk * C::CRB;
        const uint32_t base = (uint32_t)p.r0 * rb + cb0;
        const __amdgpu_buffer_rsrc_t rw = make_rsrc_uniform(p.w + base, (uint32_t)p.n * rb - base);
#pragma unroll
        for (int i = 0; i < C::WP; ++i) {
            uint32_t src = wrel[i];
            // Q8_0 chunks are always whole (K % 256 == 0 on this path)
            if constexpr (FMT == kQ4_K) src = cb0 + woff[i] < rb ? src : kOob;
            w[i] = buf_load16<false>(rw, src);
        }
        const __amdgpu_buffer_rsrc_t rf =
            make_rsrc_uniform(jb.xf, (uint32_t)xf_layout(FMT, jb.k, MT).bytes);
#pragma unroll
        for (int i = 0; i < C::FP; ++i) {
            uint32_t src;
            if constexpr (FMT == kQ8_0) {
                src = frel[i] + (uint32_t)p.chunk * (C::NBLK * 1024);
                if constexpr (C::FPIECES % 256 != 0) src = frel[i] == kOob ? kOob : src;
            } else {
                // fragment pieces advance NBLK blocks per chunk, min pieces NSB
                // super-blocks; a piece past K (partial last chunk) loads zeros
                const bool is_frag = tid + 256 * i < C::kFrag / 16;
                const uint32_t step = is_frag ? C::NBLK * 1024 : C::NSB * 512;
                const uint32_t lim = is_frag ? (uint32_t)jb.k * 32 : (uint32_t)jb.k * 2;
                const uint32_t at = (uint32_t)p.chunk * step + fpos[i];
                src = at < lim && frel[i] != kOob ? frel[i] + (uint32_t)p.chunk * step : kOob;
            }
            f[i] = buf_load16<false>(rf, src);
        }
    }

    __device__ __forceinline__ void store(uint8_t* buf, int tid) const {
#pragma unroll
        for (int i = 0; i < C::WP; ++i) {
            const int q = tid + 256 * i;
            if (q < C::WPIECES) {
                const int pr = q / (C::CRB / 16);
                const int off = (q % (C::CRB / 16)) * 16;
                *reinterpret_cast<uint4*>(buf + pr * C::RS + off) = w[i];
            }
        }
#pragma unroll
        for (int i = 0; i < C::FP; ++i) {
            const int q = tid + 256 * i;
            if (q < C::FPIECES) *reinterpret_cast<uint4*>(buf + C::kW + q * 16) = f[i];
        }
    }
};

// ---------------------------------------------------------------- main ----
// Compute one unit (chunk of a tile) from LDS; at the tile's last chunk, combine
// the K-phase partials and store.
template <int FMT, int MT, int WM>
__device__ __forceinline__ void mfma_unit(const MJobs& jobs, const MPos& cur, uint8_t* lds,
                                          uint8_t* red_lds, int batch, int lane, int wm, int wk,
                                          int j, int h, f32x4 (&acc)[MT]) {
    using C = MCfg<FMT, MT, WM>;
    constexpr int WK = C::WK;
        const MPos& jb = cur;
        mfma_chunk<FMT, MT, WM>(lds, cur.chunk * C::KC, jb.k, lane, wm, wk, j, h, acc);

        if (cur.chunk == cur.cend - 1) {
            // tile finished: sum the WK wave partials in wave order, then store
            if constexpr (WK > 1) {
                float4* red = reinterpret_cast<float4*>(red_lds);
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    red[((wk * WM + wm) * 64 + lane) * MT + t] = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
                __syncthreads();
                if (wk == 0) {
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int q = 0; q < WK; ++q) {
                            const float4 v = red[((q * WM + wm) * 64 + lane) * MT + t];
                            s += f32x4{v.x, v.y, v.z, v.w};
                        }
                        acc[t] = s;
                    }
                }
            }
            if (wk == 0) {
                const int64_t row = cur.r0 + 16 * wm + j;
                const float* inv = reinterpret_cast<const float*>(jb.xf + xf_layout(FMT, jb.k, MT).inv);
                if (row < jb.n) {
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        // D rows 4h .. 4h+3 = (batch 8t + 2h, hi/lo), (batch 8t + 2h + 1, hi/lo)
                        const int b0 = 8 * t + 2 * h;
                        float* y0 = jb.out + (int64_t)b0 * jb.ostride + row;
                        const float v0 = (acc[t][0] + acc[t][1]) * inv[b0];
                        const float v1 = (acc[t][2] + acc[t][3]) * inv[b0 + 1];
                        if (jb.add) {
                            if (b0 < batch) unsafeAtomicAdd(y0, v0);
                            if (b0 + 1 < batch) unsafeAtomicAdd(y0 + jb.ostride, v1);
                        } else {
                            if (b0 < batch) *y0 = v0;
                            if (b0 + 1 < batch) y0[jb.ostride] = v1;
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
}

template <int FMT, int MT, int WM>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(const MJobs jobs, int batch) {
    using C = MCfg<FMT, MT, WM>;
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave % WM;   // row group of this wave
    const int wk = wave / WM;   // K phase of this wave
    const int j = lane & 15;    // B-operand column = W row within the wave's 16
    const int h = lane >> 4;    // k octet (16x16x32) / k quad (16x16x16)

    // Items are handed out largest first: item blockIdx.x, then whatever the
    // work counter gives.  A workgroup asks the counter for its next item while
    // prefetching the last unit of the current one, so an item goes to the
    // workgroup that is about to be free; the answer passes through a two-slot
    // LDS ring at the following barrier.
    __shared__ int s_item[2];
    const int g = (int)gridDim.x;
    if ((int)blockIdx.x >= jobs.total_items) return;
    MPrefetch<FMT, MT, WM> pf;
    pf.job = -1;
    MPos cur = mlocate<C::RWG>(jobs, blockIdx.x);
    pf.load(jobs, cur, tid);
    bool ask = cur.chunk + 1 == cur.cend;
    if (ask && tid == 0) s_item[0] = g + atomicAdd(jobs.ctr, 1);
    pf.store(lds, tid);
    __syncthreads();
    // next item; known once cur is its item's last unit (uniform: see mlocate)
    int qnext = ask ? __builtin_amdgcn_readfirstlane(s_item[0]) : 0;
    int qslot = 1;

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One unit in flight in registers while the current one is computed from
    // one of two LDS buffers.
    int buf = 0;
    for (;;) {
        MPos nxt;
        bool more = true;
        if (cur.chunk + 1 < cur.cend) {
            nxt = cur;
            nxt.chunk = cur.chunk + 1;
        } else if (qnext < jobs.total_items) {
            nxt = mlocate<C::RWG>(jobs, qnext);
        } else {
            more = false;
        }
        ask = more && nxt.chunk + 1 == nxt.cend;
        // The counter is asked before the loads and its answer read after the
        // compute: loads complete in issue order as far as the wait counter
        // is concerned, so reading an answer issued after them would first
        // wait for the whole prefetch.  (`got` is only defined where read.)
        int got;
        if (ask && tid == 0) got = atomicAdd(jobs.ctr, 1);
        if (more) pf.load(jobs, nxt, tid);
        mfma_unit<FMT, MT, WM>(jobs, cur, lds + buf * C::kBuf, lds + 2 * C::kBuf, batch, lane, wm, wk,
                               j, h, acc);
        if (!more) break;
        if (ask && tid == 0) s_item[qslot] = g + got;
        buf ^= 1;
        pf.store(lds + buf * C::kBuf, tid);
        __syncthreads();
        if (ask) {
            qnext = __builtin_amdgcn_readfirstlane(s_item[qslot]);
            qslot ^= 1;
        }
        cur = nxt;
    }
}

int device_cus() {
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

// Longest finishing time, in units, of items handed out largest first to g
// workers that each take the next item when they finish one (list scheduling).
// cls holds (units per item, item count) pairs sorted by units, largest first.
int64_t list_makespan(const std::pair<int64_t, int64_t>* cls, int ncls, int64_t g) {
    std::map<int64_t, int64_t> load;   // finishing time -> workers
    load[0] = g;
    for (int c = 0; c < ncls; ++c) {
        int64_t rem = cls[c].second;
        while (rem > 0) {
            auto it = load.begin();
            const int64_t at = it->first, m = it->second < rem ? it->second : rem;
            if ((it->second -= m) == 0) load.erase(it);
            load[at + cls[c].first] += m;
            rem -= m;
        }
    }
    return load.rbegin()->first;
}

template <int FMT, int MT, int WM>
int mfma_blocks_per_cu() {
    using C = MCfg<FMT, MT, WM>;
    static int per_cu = 0;
    if (!per_cu) {
        if (C::kLds > 65536)
            (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_mfma_kernel<FMT, MT, WM>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gemv_mfma_kernel<FMT, MT, WM>, 256,
                                                         C::kLds) != hipSuccess || v <= 0)
            v = 1;
        per_cu = v;
    }
    return per_cu;
}

// Sums the partial results of jobs cut into more than two K parts, in part
// order: y[b][r] = part[0][b][r] + part[1][b][r] + ...
__global__ __launch_bounds__(256) void parts_sum_kernel(const MJobs jobs, int batch) {
    const MJob& jb = jobs.j[blockIdx.z];
    const int b = blockIdx.y;
    if (jb.nsplit <= 2 || b >= batch) return;
    const int64_t plane = (int64_t)batch * jb.n;
    for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < jb.n;
         r += (int64_t)gridDim.x * 256) {
        const float* p = jb.part + (int64_t)b * jb.n + r;
        float acc = p[0];
        for (int q = 1; q < jb.nsplit; ++q) acc += p[q * plane];
        jb.y[(int64_t)b * jb.ldy + r] = acc;
    }
}

// Plans the items: how many K parts each job is cut into.  Candidates: whole
// tiles; halves for the longest jobs; halves for every job of 2+ chunks; and,
// with partial-sum space, parts of at most t chunks (up to kMaxParts) for t
// from the even share of a workgroup downwards.  Each is scored by its list
// schedule (largest items first, in units of one chunk); halves must gain 3 %
// (zeroing y, the atomic adds) and deeper cuts one unit (the summing launch).
// Items are then numbered
// largest first and the activation split, main and (if needed) summing
// kernels are launched.
template <int FMT, int MT, int WM>
hipError_t launch_planned(MJobs& jobs, int batch, hipStream_t s) {
    using C = MCfg<FMT, MT, WM>;
    const int64_t slots = (int64_t)mfma_blocks_per_cu<FMT, MT, WM>() * device_cus();
    int maxc = 0;
    int64_t units = 0;
    bool parts_ok = true;
    for (int i = 0; i < jobs.count; ++i) {
        MJob& jb = jobs.j[i];
        jb.nchunk = (jb.k + C::KC - 1) / C::KC;
        jb.tiles = (int32_t)((jb.n + C::RWG - 1) / C::RWG);
        maxc = jb.nchunk > maxc ? jb.nchunk : maxc;
        units += (int64_t)jb.nchunk * jb.tiles;
        parts_ok = parts_ok && jb.part != nullptr;
    }
    // deep cuts: parts of at most `t` chunks, for t from about one
    // workgroup's even share downwards
    int64_t even = (units + slots - 1) / slots;
    int targets[8];
    int ntargets = 0;
    if (parts_ok)
        for (int64_t t = even; t >= 1 && ntargets < 8; t = t > 2 ? (t * 2) / 3 : t - 1)
            targets[ntargets++] = (int)t;
    auto parts_for = [&](int option, const MJob& jb) -> int {
        if (jb.nchunk < 2) return 1;
        if (option == 1) return jb.nchunk >= maxc ? 2 : 1;
        if (option == 2) return 2;
        if (option >= 3) {
            const int t = targets[option - 3];
            int p = (jb.nchunk + t - 1) / t;
            p = p > kMaxParts ? kMaxParts : p;
            const int cpp = (jb.nchunk + p - 1) / p;
            return (jb.nchunk + cpp - 1) / cpp;   // no empty parts
        }
        return 1;
    };
    int best = 0;
    int64_t best_cost = 0;
    for (int option = 0; option < 3 + ntargets; ++option) {
        std::pair<int64_t, int64_t> cls[kMaxJobs];
        int64_t items = 0;
        bool deep = false;
        for (int i = 0; i < jobs.count; ++i) {
            const MJob& jb = jobs.j[i];
            const int p = parts_for(option, jb);
            deep = deep || p > 2;
            cls[i].first = (jb.nchunk + p - 1) / p;
            cls[i].second = (int64_t)p * jb.tiles;
            items += cls[i].second;
        }
        std::sort(cls, cls + jobs.count,
                  [](const std::pair<int64_t, int64_t>& a, const std::pair<int64_t, int64_t>& b) {
                      return a.first > b.first;
                  });
        const int64_t cost =
            100 * (list_makespan(cls, jobs.count, items < slots ? items : slots) + (deep ? 1 : 0));
        if (option == 0 || cost < best_cost * 97 / 100) {
            best = option;
            best_cost = cost;
        }
    }
    bool any_deep = false;
    for (int i = 0; i < jobs.count; ++i) {
        MJob& jb = jobs.j[i];
        jb.nsplit = parts_for(best, jb);
        jb.cpp = (jb.nchunk + jb.nsplit - 1) / jb.nsplit;
        any_deep = any_deep || jb.nsplit > 2;
    }
    // number the largest items first (stable otherwise)
    for (int i = 1; i < jobs.count; ++i)
        for (int j = i; j > 0 && jobs.j[j].cpp > jobs.j[j - 1].cpp; --j) {
            const MJob t = jobs.j[j];
            jobs.j[j] = jobs.j[j - 1];
            jobs.j[j - 1] = t;
        }
    int total = 0;
    int64_t kmax = 0, nmax = 0;
    for (int i = 0; i < jobs.count; ++i) {
        MJob& jb = jobs.j[i];
        jb.item0 = total;
        total += jb.tiles * jb.nsplit;
        kmax = jb.k > kmax ? jb.k : kmax;
        nmax = jb.n > nmax ? jb.n : nmax;
    }
    jobs.total_items = total;
    jobs.batch = batch;
    jobs.ctr = reinterpret_cast<int32_t*>(jobs.j[0].xf + xf_layout(FMT, jobs.j[0].k, MT).ctrl);

    const dim3 pgrid((unsigned)(jobs.count * MT * 8),
                     (unsigned)((kmax / 32 + kXfragSlice - 1) / kXfragSlice));
    hipLaunchKernelGGL(xfrag_kernel<FMT>, pgrid, dim3(256), 0, s, jobs, batch, MT);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const unsigned grid = (unsigned)(total < slots ? total : slots);
    hipLaunchKernelGGL((gemv_mfma_kernel<FMT, MT, WM>), dim3(grid), dim3(256), C::kLds, s, jobs,
                       batch);
    err = hipGetLastError();
    if (err != hipSuccess || !any_deep) return err;
    const int64_t bx = (nmax + 255) / 256;
    const dim3 sgrid((unsigned)(bx < 64 ? bx : 64), (unsigned)batch, (unsigned)jobs.count);
    hipLaunchKernelGGL(parts_sum_kernel, sgrid, dim3(256), 0, s, jobs, batch);
    return hipGetLastError();
}

template <int FMT, int MT>
hipError_t launch_mt(MJobs& jobs, int batch, hipStream_t s) {
    // Rows per workgroup: 64, or 16 rows with K split over the four waves for
    // short row counts at up to 8 activation rows and no partial-sum space.  A 16-row tile loads four
    // times its weight bytes in activation fragments per chunk; it pays only
    // when 64-row tiles would leave most of the chip idle and the fragments
    // are small (one M tile).  Measured on Q4_K 9728x2560 / 2560x9728.
    int64_t rows = 0;
    for (int i = 0; i < jobs.count; ++i) rows += jobs.j[i].n;
    // With room for partial sums, K parts give the parallelism instead, and
    // 64-row tiles are kept.
    bool parts = true;
    for (int i = 0; i < jobs.count; ++i) parts = parts && jobs.j[i].part != nullptr;
    if (rows >= 8192 || MT > 1 || parts) return launch_planned<FMT, MT, 4>(jobs, batch, s);
    return launch_planned<FMT, MT, 1>(jobs, batch, s);
}

}  // namespace

size_t gemv_mfma_ws_bytes(int type, int64_t k, int batch) {
    return (size_t)xf_layout(type, k, (batch + 7) / 8).bytes;
}

size_t gemv_split_ws_bytes(int type, int64_t n, int64_t k, int batch) {
    return gemv_mfma_ws_bytes(type, k, batch) + (size_t)al256((int64_t)kMaxParts * batch * n * 4);
}

hipError_t launch_gemv_mfma(int type, const GemvDesc* descs, int count, int batch, void* ws,
                            bool parts, hipStream_t s) {
    MJobs jobs{};
    const int mt = (batch + 7) / 8;
    uint8_t* p = static_cast<uint8_t*>(ws);
    for (int i = 0; i < count; ++i) {
        const GemvDesc& d = descs[i];
        if (d.n == 0) continue;
        MJob& jb = jobs.j[jobs.count++];
        jb.w = static_cast<const uint8_t*>(d.w);
        jb.x = d.x;
        jb.y = d.y;
        jb.xf = p;
        jb.n = d.n;
        jb.ldx = d.ldx;
        jb.ldy = d.ldy;
        jb.rb = row_bytes(type, d.k);
        jb.k = (int32_t)d.k;
        p += gemv_mfma_ws_bytes(type, d.k, batch);
        if (parts) {
            jb.part = reinterpret_cast<float*>(p);
            p += gemv_split_ws_bytes(type, d.n, d.k, batch) - gemv_mfma_ws_bytes(type, d.k, batch);
        }
    }
    if (jobs.count == 0) return hipSuccess;
    if (type == kQ4_K)
        return mt == 1 ? launch_mt<kQ4_K, 1>(jobs, batch, s) : launch_mt<kQ4_K, 2>(jobs, batch, s);
    return mt == 1 ? launch_mt<kQ8_0, 1>(jobs, batch, s) : launch_mt<kQ8_0, 2>(jobs, batch, s);
}

}  // namespace ggq
