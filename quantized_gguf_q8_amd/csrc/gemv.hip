// gemv.hip -- quant_gemv: decode-time matrix-vector product over Q8_0 / Q4_K rows,
// batch 1..16, weights decoded on the fly and never written back (Phobos README,
// "Inference").  The workgroup algorithm is in gemv_core.h.
#include "gemv_core.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

struct StoreEpi {
    float* y;
    int64_t ldy;
    __device__ void operator()(int b, int64_t r, const float (&v)[1]) const {
        y[(int64_t)b * ldy + r] = v[0];
    }
};

template <int FMT, int NB, int ROWS>
__global__ __launch_bounds__(256) void gemv_kernel(const uint8_t* __restrict__ w, int64_t n, int k,
                                                   int64_t rbytes, const float* __restrict__ x,
                                                   int64_t ldx, float* __restrict__ y,
                                                   int64_t ldy, int batch) {
    extern __shared__ __align__(16) uint8_t lds[];
    const uint8_t* wm[1] = {w};
    const float* xr[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) xr[b] = x + (int64_t)b * ldx;
    StoreEpi epi{y, ldy};
    gemv_tile<FMT, NB, ROWS, 1>(lds, wm, n, k, rbytes, xr, batch, (int64_t)blockIdx.x * ROWS, epi);
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

template <int FMT, int NB, int ROWS>
hipError_t launch_cfg(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const float* x,
                      int64_t ldx, float* y, int64_t ldy, int batch, hipStream_t s) {
    using C = GemvCfg<FMT, NB, ROWS, 1>;
    dim3 grid((unsigned)((n + ROWS - 1) / ROWS));
    hipLaunchKernelGGL((gemv_kernel<FMT, NB, ROWS>), grid, dim3(256), C::kLds, s, w, n, (int)k, rb,
                       x, ldx, y, ldy, batch);
    return hipGetLastError();
}

template <int FMT, int NB>
hipError_t launch_nb(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const float* x,
                     int64_t ldx, float* y, int64_t ldy, int batch, hipStream_t s) {
    const int rows = gemv_rows_for(NB, k);
    if constexpr (2 * NB <= 8)
        if (rows == 8) return launch_cfg<FMT, NB, 8>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    if constexpr (2 * NB <= 16)
        if (rows == 16) return launch_cfg<FMT, NB, 16>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    if constexpr (2 * NB <= 32)
        if (rows == 32) return launch_cfg<FMT, NB, 32>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    return launch_cfg<FMT, NB, 64>(w, n, k, rb, x, ldx, y, ldy, batch, s);
}

template <int FMT>
hipError_t launch_fmt(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const float* x,
                      int64_t ldx, float* y, int64_t ldy, int batch, hipStream_t s) {
    if (batch <= 1) return launch_nb<FMT, 1>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    if (batch <= 2) return launch_nb<FMT, 2>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    if (batch <= 4) return launch_nb<FMT, 4>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    if (batch <= 8) return launch_nb<FMT, 8>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    return launch_nb<FMT, 16>(w, n, k, rb, x, ldx, y, ldy, batch, s);
}

template <int NB>
hipError_t launch_generic(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const float* x,
                          int64_t ldx, float* y, int64_t ldy, int batch, hipStream_t s) {
    hipLaunchKernelGGL((gemv_q8_0_generic<NB>), dim3((unsigned)n), dim3(64), 0, s, w, (int)k, rb,
                       x, ldx, y, ldy, batch);
    return hipGetLastError();
}

}  // namespace

int64_t row_bytes(int type, int64_t k) {
    return type == kQ8_0 ? k / 32 * kQ8Bytes : k / 256 * kQ4Bytes;
}

hipError_t launch_gemv(int type, const uint8_t* w, int64_t n, int64_t k, const float* x,
                       int64_t ldx, float* y, int64_t ldy, int batch, hipStream_t s) {
    const int64_t rb = row_bytes(type, k);
    if (type == kQ4_K) return launch_fmt<kQ4_K>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    if (k % 256 == 0) return launch_fmt<kQ8_0>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    if (batch <= 4) return launch_generic<4>(w, n, k, rb, x, ldx, y, ldy, batch, s);
    return launch_generic<16>(w, n, k, rb, x, ldx, y, ldy, batch, s);
}

}  // namespace ggq
