// gemv_mfma.hip -- batched decode GEMV (batch 2..16) on the matrix cores.
//
// Same product as quant_gemv (Phobos README, "Inference"); the operand
// conversions and the per-chunk MFMA arithmetic are in gemv_mfma_core.h.
//
// Work decomposition: a workgroup (4 waves) owns 16*WM rows; each wave owns 16
// rows (the 16 columns of the B operand) and every WK-th block of each K chunk
// (WM*WK = 4).  Chunks of weights and activation fragments are staged through LDS
// with the same register-prefetch pipeline as the VALU path; workgroups are
// persistent over row tiles.  The WK partials of a tile are summed in LDS in wave
// order at the end of its K walk.
#include "gemv_mfma_core.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

struct MPos {
    int tile, job, chunk;
    int64_t r0;
};

template <int RWG>
__device__ __forceinline__ MPos mlocate(const MJobs& jobs, int tile, int chunk) {
    int j = 0;
    while (j + 1 < jobs.count && tile >= jobs.j[j + 1].tile0) ++j;
    MPos p;
    p.tile = tile;
    p.job = j;
    p.chunk = chunk;
    p.r0 = (int64_t)(tile - jobs.j[j].tile0) * RWG;
    return p;
}

template <int FMT, int MT, int WM>
struct MPrefetch {
    using C = MCfg<FMT, MT, WM>;
    uint4 w[C::WP];
    uint4 f[C::FP];

    // Out-of-range pieces (rows past N, bytes past a row, blocks past K) load
    // from an offset beyond the descriptor and come back as zeros.
    __device__ __forceinline__ void load(const MJobs& jobs, const MPos& p, int tid) {
        const MJob& jb = jobs.j[p.job];
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(jb.w, (uint32_t)(jb.n * jb.rb));
        const uint32_t rb = (uint32_t)jb.rb;
        const uint32_t cb0 = (uint32_t)p.chunk * C::CRB;
        const uint32_t base = (uint32_t)p.r0 * rb + cb0;
#pragma unroll
        for (int i = 0; i < C::WP; ++i) {
            const int q = tid + 256 * i;
            const uint32_t pr = (uint32_t)q / (C::CRB / 16);
            const uint32_t off = ((uint32_t)q % (C::CRB / 16)) * 16;
            const bool ok = q < C::WPIECES && cb0 + off < rb;
            w[i] = buf_load16<true>(rw, ok ? base + pr * rb + off : kOob);
        }
        const XfLayout L = xf_layout(FMT, jb.k, MT);
        const __amdgpu_buffer_rsrc_t rf = make_rsrc(jb.xf, (uint32_t)L.bytes);
        const int nblk = jb.k / 32;
        const int nsb = jb.k / 256;
#pragma unroll
        for (int i = 0; i < C::FP; ++i) {
            const int q = tid + 256 * i;
            const int o = q * 16;  // byte offset inside this chunk's fragment staging
            uint32_t src = kOob;
            if (q < C::FPIECES) {
                if (o < C::kFrag) {
                    const int t = o / (C::NBLK * 1024);
                    const int rem = o % (C::NBLK * 1024);
                    const int blk = p.chunk * C::NBLK + rem / 1024;
                    if (blk < nblk)
                        src = (uint32_t)(L.frag + ((int64_t)t * nblk + blk) * 1024 + rem % 1024);
                } else if constexpr (FMT == kQ4_K) {
                    const int o2 = o - C::kFrag;
                    const int t = o2 / (C::NSB * 512);
                    const int rem = o2 % (C::NSB * 512);
                    const int sb = p.chunk * C::NSB + rem / 512;
                    if (sb < nsb) src = (uint32_t)(L.mins + ((int64_t)t * nsb + sb) * 512 + rem % 512);
                }
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
template <int RWG>
__device__ __forceinline__ bool mnext(const MJobs& jobs, const MPos& p, MPos& q) {
    if (p.chunk + 1 < jobs.j[p.job].nchunk) {
        q = p;
        q.chunk = p.chunk + 1;
        return true;
    }
    // Workgroup b takes tile b in round 0, G-1-b in round 1, b in round 2, ...
    // (G = grid size): with the longest jobs numbered first, the workgroups that
    // drew a long tile in round 0 are the last to be served in round 1.
    const int g = (int)gridDim.x;
    const int r = p.tile / g;
    const int b = (r & 1) ? g - 1 - p.tile % g : p.tile % g;
    const int tn = (r + 1) * g + (((r + 1) & 1) ? g - 1 - b : b);
    if (tn >= jobs.total_tiles) return false;
    q = mlocate<RWG>(jobs, tn, 0);
    return true;
}

// Compute one unit (chunk of a tile) from LDS; at the tile's last chunk, combine
// the K-phase partials and store.
template <int FMT, int MT, int WM>
__device__ __forceinline__ void mfma_unit(const MJobs& jobs, const MPos& cur, uint8_t* lds,
                                          uint8_t* red_lds, int batch, int lane, int wm, int wk,
                                          int j, int h, f32x4 (&acc)[MT]) {
    using C = MCfg<FMT, MT, WM>;
    constexpr int WK = C::WK;
        const MJob& jb = jobs.j[cur.job];
        mfma_chunk<FMT, MT, WM>(lds, cur.chunk * C::KC, jb.k, lane, wm, wk, j, h, acc);

        if (cur.chunk == jb.nchunk - 1) {
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
                        if (b0 < batch) jb.y[(int64_t)b0 * jb.ldy + row] = (acc[t][0] + acc[t][1]) * inv[b0];
                        if (b0 + 1 < batch) jb.y[(int64_t)(b0 + 1) * jb.ldy + row] = (acc[t][2] + acc[t][3]) * inv[b0 + 1];
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

    if ((int)blockIdx.x >= jobs.total_tiles) return;
    MPrefetch<FMT, MT, WM> pf;
    MPos cur = mlocate<C::RWG>(jobs, blockIdx.x, 0);
    pf.load(jobs, cur, tid);
    pf.store(lds, tid);
    __syncthreads();

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One unit in flight in registers while the current one is computed from
    // one of two LDS buffers.
    int buf = 0;
    for (;;) {
        MPos nxt;
        const bool more = mnext<C::RWG>(jobs, cur, nxt);
        if (more) pf.load(jobs, nxt, tid);
        mfma_unit<FMT, MT, WM>(jobs, cur, lds + buf * C::kBuf, lds + 2 * C::kBuf, batch, lane, wm, wk,
                               j, h, acc);
        if (!more) break;
        buf ^= 1;
        pf.store(lds + buf * C::kBuf, tid);
        __syncthreads();
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

template <int FMT, int MT, int WM>
hipError_t launch_main(MJobs& jobs, int batch, hipStream_t s) {
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
    // number the tiles of the longest-K jobs first (stable order otherwise)
    for (int i = 1; i < jobs.count; ++i)
        for (int j = i; j > 0 && jobs.j[j].k > jobs.j[j - 1].k; --j) {
            const MJob t = jobs.j[j];
            jobs.j[j] = jobs.j[j - 1];
            jobs.j[j - 1] = t;
        }
    int total = 0;
    for (int i = 0; i < jobs.count; ++i) {
        MJob& jb = jobs.j[i];
        jb.nchunk = (jb.k + C::KC - 1) / C::KC;
        jb.tile0 = total;
        jb.tiles = (int32_t)((jb.n + C::RWG - 1) / C::RWG);
        total += jb.tiles;
    }
    jobs.total_tiles = total;
    const int64_t slots = (int64_t)per_cu * device_cus();
    const unsigned grid = (unsigned)(total < slots ? total : slots);
    hipLaunchKernelGGL((gemv_mfma_kernel<FMT, MT, WM>), dim3(grid), dim3(256), C::kLds, s, jobs,
                       batch);
    return hipGetLastError();
}

template <int FMT, int MT>
hipError_t launch_mt(MJobs& jobs, int batch, hipStream_t s) {
    // Rows per workgroup: 64 when there are enough row tiles to fill the chip,
    // otherwise 16 rows with K split over the four waves.
    int64_t rows = 0;
    for (int i = 0; i < jobs.count; ++i) rows += jobs.j[i].n;
    if (rows >= 64 * 512) return launch_main<FMT, MT, 4>(jobs, batch, s);
    return launch_main<FMT, MT, 1>(jobs, batch, s);
}

}  // namespace

size_t gemv_mfma_ws_bytes(int type, int64_t k, int batch) {
    return (size_t)xf_layout(type, k, (batch + 7) / 8).bytes;
}

hipError_t launch_gemv_mfma(int type, const GemvDesc* descs, int count, int batch, void* ws,
                            hipStream_t s) {
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
    }
    if (jobs.count == 0) return hipSuccess;
    int64_t kmax = 0;
    for (int i = 0; i < jobs.count; ++i) kmax = jobs.j[i].k > kmax ? jobs.j[i].k : kmax;
    const dim3 pgrid((unsigned)(jobs.count * mt * 8),
                     (unsigned)((kmax / 32 + kXfragSlice - 1) / kXfragSlice));
    if (type == kQ4_K)
        hipLaunchKernelGGL(xfrag_kernel<kQ4_K>, pgrid, dim3(256), 0, s, jobs, batch, mt);
    else
        hipLaunchKernelGGL(xfrag_kernel<kQ8_0>, pgrid, dim3(256), 0, s, jobs, batch, mt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (type == kQ4_K)
        return mt == 1 ? launch_mt<kQ4_K, 1>(jobs, batch, s) : launch_mt<kQ4_K, 2>(jobs, batch, s);
    return mt == 1 ? launch_mt<kQ8_0, 1>(jobs, batch, s) : launch_mt<kQ8_0, 2>(jobs, batch, s);
}

}  // namespace ggq
