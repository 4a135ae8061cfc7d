// gemv.hip -- quant_gemv / quant_gemv_grouped: decode-time matrix-vector products
// over Q8_0 / Q4_K rows, batch 1..16, weights decoded on the fly and never
// written back (Phobos README, "Inference").  A grouped call runs several
// matrices (e.g. every projection of a decoder layer, README "Components":
// kernel fusion) in one launch.
//
// Streaming structure (gfx950, 256-thread workgroups, wave64):
//  * Work unit = (matrix, tile of ROWS rows, K chunk of KC = 64*SL weights),
//    SL = 256/ROWS.  Thread (row rl, slice s), slice fastest, owns 64 weights of
//    its row per chunk: two Q8_0 blocks or a 64-weight quarter of a Q4_K
//    super-block.
//  * Workgroups are persistent: each walks its share of the unit stream.  While
//    it computes unit u from one LDS buffer, the 16-byte global loads of unit
//    u+1 (weights, coalesced along each row, and the activation chunk) are
//    already in flight into registers; they land in the other LDS buffer after
//    the compute, so one barrier per unit suffices and HBM never waits for the
//    arithmetic.
//  * A thread decodes its 64 weights once and applies them to every batch row.
//  * The SL slices of a row sit in one wave (slice fastest, SL divides 64), so
//    a row's partials are combined with a fixed butterfly of lane shuffles:
//    deterministic, no LDS round trip.
//  * Q4_K uses the factored form per 32-weight sub-block j,
//        d*sc_j * sum q_c x_c - dmin*m_j * sum x_c,
//    with the activation sums formed once per chunk while staging.
#include "gemv_core.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

constexpr int kMaxJobs = 16;

struct GemvJob {
    const uint8_t* w;
    const float* x;
    float* y;
    int64_t n;
    int64_t ldx;
    int64_t ldy;
    int64_t rb;      // bytes per row
    int32_t k;
    int32_t nchunk;  // K chunks per tile
    int32_t tile0;   // first tile of this job in the grouped tile index space
    int32_t tiles;
};

struct GemvJobs {
    GemvJob j[kMaxJobs];
    int32_t count;
    int32_t total_tiles;
};

template <int FMT, int NB, int ROWS>
struct StreamCfg {
    using Base = GemvCfg<FMT, NB, ROWS, 1>;
    static constexpr int SL = Base::SL;
    static constexpr int KC = Base::KC;
    static constexpr int CRB = Base::CRB;
    static constexpr int WRS = Base::WRS;
    static constexpr int XSS = Base::XSS;
    static constexpr int XBS = Base::XBS;
    static constexpr int PPR = CRB / 16;               // 16-byte pieces per row chunk
    static constexpr int WPIECES = ROWS * PPR;
    static constexpr int WP = (WPIECES + 255) / 256;   // per thread
    static constexpr int XPIECES = NB * KC / 4;        // float4 pieces of the x chunk
    static constexpr int XP = (XPIECES + 255) / 256;
    static constexpr int kWBytes = ROWS * WRS;
    static constexpr int kXBytes = NB * XBS * 4;
    static constexpr int kSumBytes = FMT == kQ4_K ? NB * SL * 2 * 4 : 0;
    static constexpr int kXBuf = kXBytes + kSumBytes;
    // one weight buffer, two activation buffers
    static constexpr int kLds = kWBytes + 2 * kXBuf;
};

// A unit is one K chunk of one tile.  A workgroup takes tiles bid, bid+G, ...
// and walks each tile's chunks in order, so a row's partial sums stay in the
// registers of the threads that own it.
struct UnitPos {
    int tile;   // grouped tile index
    int job;
    int64_t r0;
    int chunk;
};

__device__ __forceinline__ UnitPos locate(const GemvJobs& jobs, int tile, int chunk, int rows) {
    int j = 0;
    while (j + 1 < jobs.count && tile >= jobs.j[j + 1].tile0) ++j;
    UnitPos p;
    p.tile = tile;
    p.job = j;
    p.r0 = (int64_t)(tile - jobs.j[j].tile0) * rows;
    p.chunk = chunk;
    return p;
}

template <int ROWS>
__device__ __forceinline__ bool next_unit(const GemvJobs& jobs, const UnitPos& p, UnitPos& q) {
    if (p.chunk + 1 < jobs.j[p.job].nchunk) {
        q = p;
        q.chunk = p.chunk + 1;
        return true;
    }
    const int tn = p.tile + (int)gridDim.x;
    if (tn >= jobs.total_tiles) return false;
    q = locate(jobs, tn, 0, ROWS);
    return true;
}

// Registers holding the next unit's bytes between its global loads and its LDS
// stores.  Pieces outside the matrix, past a row's end or past K are loaded
// from an out-of-range buffer offset and come back as zeros.
template <int FMT, int NB, int ROWS>
struct Prefetch {
    using C = StreamCfg<FMT, NB, ROWS>;
    uint4 w[C::WP];
    uint4 x[C::XP];

    __device__ __forceinline__ void load_w(const GemvJob& jb, const UnitPos& p, int tid) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(jb.w, (uint32_t)(jb.n * jb.rb));
        const uint32_t cb0 = (uint32_t)p.chunk * C::CRB;
        const uint32_t rb = (uint32_t)jb.rb;
        const uint32_t base = (uint32_t)p.r0 * rb + cb0;
#pragma unroll
        for (int i = 0; i < C::WP; ++i) {
            const int q = tid + 256 * i;
            const uint32_t pr = (uint32_t)q / C::PPR;
            const uint32_t off = ((uint32_t)q % C::PPR) * 16;
            const bool ok = q < C::WPIECES && cb0 + off < rb;
            w[i] = buf_load16<true>(r, ok ? base + pr * rb + off : kOob);
        }
    }

    __device__ __forceinline__ void load_x(const GemvJob& jb, const UnitPos& p, int batch,
                                           int tid) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(jb.x, (uint32_t)(batch * jb.ldx * 4));
        const int k0 = p.chunk * C::KC;
#pragma unroll
        for (int i = 0; i < C::XP; ++i) {
            const int q = tid + 256 * i;
            const int b = q / (C::KC / 4);
            const int pos = (q % (C::KC / 4)) * 4;
            const bool ok = q < C::XPIECES && k0 + pos < jb.k;
            x[i] = buf_load16<false>(r, ok ? (uint32_t)((b * jb.ldx + k0 + pos) * 4) : kOob);
        }
    }

    __device__ __forceinline__ void store_w(uint8_t* lw, int tid) const {
#pragma unroll
        for (int i = 0; i < C::WP; ++i) {
            const int q = tid + 256 * i;
            if (q < C::WPIECES) {
                const int pr = q / C::PPR;
                const int off = (q % C::PPR) * 16;
                *reinterpret_cast<uint4*>(lw + pr * C::WRS + off) = w[i];
            }
        }
    }

    __device__ __forceinline__ void store_x(uint8_t* xbuf, int tid) const {
        float* lx = reinterpret_cast<float*>(xbuf);
        float* lsum = reinterpret_cast<float*>(xbuf + C::kXBytes);
#pragma unroll
        for (int i = 0; i < C::XP; ++i) {
            const int q = tid + 256 * i;
            if (C::XPIECES % 256 == 0 || q < C::XPIECES) {  // whole waves only
                const int b = q / (C::KC / 4);
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

template <int FMT, int NB, int ROWS>
__device__ __forceinline__ void stream_compute(const GemvJobs& jobs, const UnitPos& cur,
                                               const uint8_t* lw, const uint8_t* xbuf, int batch,
                                               int s, int rl, float (&acc)[NB]) {
    using C = StreamCfg<FMT, NB, ROWS>;
    constexpr int SL = C::SL;
    const GemvJob& jb = jobs.j[cur.job];
    const float* lx = reinterpret_cast<const float*>(xbuf);
    const float* lsum = reinterpret_cast<const float*>(xbuf + C::kXBytes);
    const int k0 = cur.chunk * C::KC;
    if (cur.r0 + rl < jb.n && k0 + s * 64 < jb.k) {
        float f0[32], f1[32];
        float sa0, sa1, mb0, mb1;
        decode_unit<FMT>(lw + rl * C::WRS, s, f0, f1, sa0, sa1, mb0, mb1);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < batch) {
                const float4* xv = reinterpret_cast<const float4*>(lx + b * C::XBS + s * C::XSS);
                float p0[4] = {0.f, 0.f, 0.f, 0.f}, p1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float4 a = xv[i];
                    float4 e = xv[8 + i];
                    p0[i & 3] += f0[4 * i] * a.x + f0[4 * i + 1] * a.y + f0[4 * i + 2] * a.z +
                                 f0[4 * i + 3] * a.w;
                    p1[i & 3] += f1[4 * i] * e.x + f1[4 * i + 1] * e.y + f1[4 * i + 2] * e.z +
                                 f1[4 * i + 3] * e.w;
                }
                float t = sa0 * ((p0[0] + p0[1]) + (p0[2] + p0[3])) +
                          sa1 * ((p1[0] + p1[1]) + (p1[2] + p1[3]));
                if constexpr (FMT == kQ4_K) {
                    const float* xs = lsum + (b * SL + s) * 2;
                    t -= mb0 * xs[0] + mb1 * xs[1];
                }
                acc[b] += t;
            }
        }
    }
    if (cur.chunk == jb.nchunk - 1) {
        // row finished: butterfly over the SL slice lanes of this row
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int o = 1; o < SL; o <<= 1) acc[b] += __shfl_xor(acc[b], o, 64);
        }
        if (s == 0 && cur.r0 + rl < jb.n) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < batch) jb.y[b * jb.ldy + cur.r0 + rl] = acc[b];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.f;
    }
}

// One unit in flight in registers while the current one is computed from LDS.
// Weights have one LDS buffer, refilled behind a barrier once every wave is
// done with it: the second buffer of a double-buffered layout let only three
// workgroups share a compute unit instead of four (38.5 against 34.7 us for
// the Q8_0 layer set at batch 1), and the unit in flight in registers already
// hides the load.  The activation chunk is double-buffered and staged only when
// the (matrix, chunk) changes -- for K <= KC that is once per matrix.
template <int FMT, int NB, int ROWS>
__global__ __launch_bounds__(256) void gemv_stream_kernel(const GemvJobs jobs, int batch) {
    using C = StreamCfg<FMT, NB, ROWS>;
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t* lw0 = lds;
    uint8_t* lx0 = lds + C::kWBytes;
    const int tid = threadIdx.x;
    const int s = tid % C::SL;
    const int rl = tid / C::SL;

    if ((int)blockIdx.x >= jobs.total_tiles) return;
    Prefetch<FMT, NB, ROWS> pf;
    UnitPos cur = locate(jobs, blockIdx.x, 0, ROWS);
    pf.load_w(jobs.j[cur.job], cur, tid);
    pf.load_x(jobs.j[cur.job], cur, batch, tid);
    pf.store_w(lw0, tid);
    pf.store_x(lx0, tid);
    int xjob = cur.job, xchunk = cur.chunk, xb = 0;
    __syncthreads();

    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;

    for (;;) {
        UnitPos nxt;
        const bool more = next_unit<ROWS>(jobs, cur, nxt);
        bool newx = false;
        if (more) {
            pf.load_w(jobs.j[nxt.job], nxt, tid);
            newx = nxt.job != xjob || nxt.chunk != xchunk;
            if (newx) pf.load_x(jobs.j[nxt.job], nxt, batch, tid);
        }
        stream_compute<FMT, NB, ROWS>(jobs, cur, lw0, lx0 + xb * C::kXBuf, batch, s, rl, acc);
        if (!more) break;
        __syncthreads();   // every wave is done with the weight buffer
        pf.store_w(lw0, tid);
        if (newx) {
            xb ^= 1;
            pf.store_x(lx0 + xb * C::kXBuf, tid);
            xjob = nxt.job;
            xchunk = nxt.chunk;
        }
        __syncthreads();
        cur = nxt;
    }
}

// Fallback for Q8_0 rows that are not whole 16-byte pieces (K % 256 != 0): one
// wave per row, one lane per 32-weight block, halfword loads.
template <int NB>
__global__ __launch_bounds__(64) void gemv_q8_0_generic(const uint8_t* __restrict__ w, int k,
                                                        int64_t rbytes,
                                                        const float* __restrict__ x, int64_t ldx,
                                                        float* __restrict__ y, int64_t ldy,
                                                        int batch) {
    const int64_t r = blockIdx.x;
    const int lane = threadIdx.x;
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
    const int nb = k / 32;
    for (int blk = lane; blk < nb; blk += 64) {
        const uint16_t* h =
            reinterpret_cast<const uint16_t*>(w + r * rbytes + (int64_t)blk * kQ8Bytes);
        float d = half_bits_to_float(h[0]);
        float f[32];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t v = h[1 + i];
            f[2 * i] = sbyte_f(v, 0);
            f[2 * i + 1] = sbyte_f(v, 1);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < batch) {
                const float* xb = x + (int64_t)b * ldx + blk * 32;
                float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 32; ++i) p[i & 3] += f[i] * xb[i];
                acc[b] += d * ((p[0] + p[1]) + (p[2] + p[3]));
            }
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float t = wave_sum(acc[b]);
        if (lane == 0 && b < batch) y[(int64_t)b * ldy + r] = t;
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

// Resident workgroups of one tile height on the whole device.
template <int FMT, int NB, int ROWS>
int64_t stream_slots() {
    using C = StreamCfg<FMT, NB, ROWS>;
    static int per_cu = 0;
    if (!per_cu) {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gemv_stream_kernel<FMT, NB, ROWS>, 256,
                                                         C::kLds) != hipSuccess || v <= 0)
            v = 2;
        per_cu = v;
    }
    return (int64_t)per_cu * device_cus();
}

// Units on the longest workgroup's path for one matrix: the tiles it walks
// times the K chunks of each.  Every unit waits for its own loads, so this is
// the number of dependent HBM round trips a small launch lasts.
template <int FMT, int NB, int ROWS>
int64_t stream_chain(const GemvJob& jb) {
    using C = StreamCfg<FMT, NB, ROWS>;
    const int64_t tiles = (jb.n + ROWS - 1) / ROWS, slots = stream_slots<FMT, NB, ROWS>();
    return (tiles + slots - 1) / slots * ((jb.k + C::KC - 1) / C::KC);
}

template <int FMT, int NB, int ROWS>
hipError_t launch_stream(GemvJobs& jobs, int batch, hipStream_t s) {
    using C = StreamCfg<FMT, NB, ROWS>;
    int total = 0;
    for (int i = 0; i < jobs.count; ++i) {
        GemvJob& jb = jobs.j[i];
        const int64_t tiles = (jb.n + ROWS - 1) / ROWS;
        jb.nchunk = (jb.k + C::KC - 1) / C::KC;
        jb.tile0 = total;
        jb.tiles = (int32_t)tiles;
        total += jb.tiles;
    }
    jobs.total_tiles = total;
    if (total == 0) return hipSuccess;
    const int64_t slots = stream_slots<FMT, NB, ROWS>();
    const unsigned grid = (unsigned)(total < slots ? total : slots);
    hipLaunchKernelGGL((gemv_stream_kernel<FMT, NB, ROWS>), dim3(grid), dim3(256), C::kLds, s, jobs,
                       batch);
    return hipGetLastError();
}

template <int FMT, int NB>
hipError_t launch_nb(GemvJobs& jobs, int batch, int64_t kmin, hipStream_t s) {
    int rows = gemv_rows_for(NB, kmin);
    if (jobs.count == 1) {
        // One matrix: a taller tile (fewer tiles, more K chunks each) when that
        // shortens the longest workgroup's chain of units, e.g. Q4_K 9728x2560
        // at batch 1: 1216 8-row tiles on 1024 resident workgroups walk up to
        // 2 x 2 units, 608 16-row tiles 1 x 3 (8.97 against 8.06 us).
        auto chain = [&](int r) -> int64_t {
            if constexpr (2 * NB <= 8)
                if (r == 8) return stream_chain<FMT, NB, 8>(jobs.j[0]);
            if constexpr (2 * NB <= 16)
                if (r == 16) return stream_chain<FMT, NB, 16>(jobs.j[0]);
            if constexpr (2 * NB <= 32)
                if (r == 32) return stream_chain<FMT, NB, 32>(jobs.j[0]);
            return stream_chain<FMT, NB, 64>(jobs.j[0]);
        };
        int64_t best = chain(rows);
        for (int r = rows * 2; r <= 64; r *= 2) {
            const int64_t c = chain(r);
            if (c < best) {
                best = c;
                rows = r;
            }
        }
    }
    if constexpr (2 * NB <= 8)
        if (rows == 8) return launch_stream<FMT, NB, 8>(jobs, batch, s);
    if constexpr (2 * NB <= 16)
        if (rows == 16) return launch_stream<FMT, NB, 16>(jobs, batch, s);
    if constexpr (2 * NB <= 32)
        if (rows == 32) return launch_stream<FMT, NB, 32>(jobs, batch, s);
    return launch_stream<FMT, NB, 64>(jobs, batch, s);
}

template <int FMT>
hipError_t launch_fmt(GemvJobs& jobs, int batch, int64_t kmin, hipStream_t s) {
    if (batch <= 1) return launch_nb<FMT, 1>(jobs, batch, kmin, s);
    if (batch <= 2) return launch_nb<FMT, 2>(jobs, batch, kmin, s);
    if (batch <= 4) return launch_nb<FMT, 4>(jobs, batch, kmin, s);
    if (batch <= 8) return launch_nb<FMT, 8>(jobs, batch, kmin, s);
    return launch_nb<FMT, 16>(jobs, batch, kmin, s);
}

template <int NB>
hipError_t launch_generic(const GemvDesc& d, int batch, hipStream_t s) {
    const int64_t rb = row_bytes(kQ8_0, d.k);
    hipLaunchKernelGGL((gemv_q8_0_generic<NB>), dim3((unsigned)d.n), dim3(64), 0, s,
                       static_cast<const uint8_t*>(d.w), (int)d.k, rb, d.x, d.ldx, d.y, d.ldy,
                       batch);
    return hipGetLastError();
}

}  // namespace

int64_t row_bytes(int type, int64_t k) {
    return type == kQ8_0 ? k / 32 * kQ8Bytes : k / 256 * kQ4Bytes;
}

int gemv_max_group() { return kMaxJobs; }

hipError_t launch_gemv_group(int type, const GemvDesc* descs, int count, int batch,
                             hipStream_t s) {
    GemvJobs jobs{};
    int64_t kmin = INT64_MAX;
    for (int i = 0; i < count; ++i) {
        const GemvDesc& d = descs[i];
        if (d.n == 0) continue;
        if (type == kQ8_0 && d.k % 256 != 0) {
            hipError_t e = batch <= 4 ? launch_generic<4>(d, batch, s) : launch_generic<16>(d, batch, s);
            if (e != hipSuccess) return e;
            continue;
        }
        GemvJob& jb = jobs.j[jobs.count++];
        jb.w = static_cast<const uint8_t*>(d.w);
        jb.x = d.x;
        jb.y = d.y;
        jb.n = d.n;
        jb.ldx = d.ldx;
        jb.ldy = d.ldy;
        jb.rb = row_bytes(type, d.k);
        jb.k = (int32_t)d.k;
        if (d.k < kmin) kmin = d.k;
    }
    if (jobs.count == 0) return hipSuccess;
    if (type == kQ4_K) return launch_fmt<kQ4_K>(jobs, batch, kmin, s);
    return launch_fmt<kQ8_0>(jobs, batch, kmin, s);
}

hipError_t launch_gemv(int type, const uint8_t* w, int64_t n, int64_t k, const float* x,
                       int64_t ldx, float* y, int64_t ldy, int batch, hipStream_t s) {
    GemvDesc d{w, n, k, x, ldx, y, ldy};
    return launch_gemv_group(type, &d, 1, batch, s);
}

}  // namespace ggq
