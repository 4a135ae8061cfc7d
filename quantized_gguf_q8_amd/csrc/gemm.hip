// gemm.hip -- quant_gemm: prompt-batch product C[M][N] = A[M][K] * W[N][K]^T with
// W in Q8_0 / Q4_K blocks (phobos-bench pp<N>, Phobos README "Command-Line
// Tools"; the pages report prompt processing as their weaker path).
//
// This is the one dense contraction on the path, so it runs on the matrix cores:
//  1. prep : A fp32 -> bf16 (round to nearest even) into the workspace, rows
//            padded with zeros to a multiple of 64 columns.
//  2. main : 256-thread workgroups own a BM x BN tile of C (BM = 128, four waves
//            of 32 rows each, BN = 16*NT).  Per 64-wide K step the A tile is
//            copied to LDS and the W tile is decoded from its blocks straight to
//            bf16 in LDS (each weight decoded once per workgroup and reused by all
//            BM rows), then every wave runs v_mfma_f32_16x16x32_bf16 over its
//            32 x BN sub-tile with fp32 accumulators.
// Rounding: A and the decoded weights are each rounded once to bf16 (relative
// error <= 2^-9 each); products and sums are fp32.
#include "ggq_device.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kBM = 128;
constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 8;  // bf16 per LDS row (16-byte pad)

inline int64_t kpad(int64_t k) { return (k + kBK - 1) / kBK * kBK; }

__global__ __launch_bounds__(256) void prep_bf16_kernel(const float* __restrict__ a, int64_t lda,
                                                        int64_t m, int64_t k, int64_t kp,
                                                        uint16_t* __restrict__ out) {
    const int64_t q = kp / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= m * q) return;
    const int64_t row = i / q;
    const int64_t col = (i % q) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col < k) v = *reinterpret_cast<const float4*>(a + row * lda + col);
    uint2 o;
    o.x = pack_bf16x2(v.x, v.y);
    o.y = pack_bf16x2(v.z, v.w);
    *reinterpret_cast<uint2*>(out + row * kp + col) = o;
}

// Decode 32 weights of W row `nrow` for K step k0 into bf16 LDS row `dst`.
// Thread half h selects which 32: Q8_0 block (k0/32 + h); Q4_K quant bytes
// 16h..16h+15 of the step's 64-weight group (16 low-nibble and 16 high-nibble
// weights, at local columns 16h.. and 32+16h..).
template <int FMT>
__device__ __forceinline__ void decode_w32(const uint8_t* __restrict__ w, int64_t nrow, bool ok,
                                           int64_t rb, int64_t k, int k0, int h, uint16_t* dst) {
    uint32_t o[16];
    if constexpr (FMT == kQ8_0) {
        const int64_t kb = k0 / 32 + h;
        if (ok && kb < k / 32) {
            const uint16_t* p = reinterpret_cast<const uint16_t*>(w + nrow * rb + kb * kQ8Bytes);
            float d = half_bits_to_float(p[0]);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t v = p[1 + i];
                o[i] = pack_bf16x2(d * sbyte_f(v, 0), d * sbyte_f(v, 1));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] = 0;
        }
        uint4* d4 = reinterpret_cast<uint4*>(dst + 32 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) d4[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    } else {
        if (ok) {
            const uint8_t* sb = w + nrow * rb + (int64_t)(k0 / 256) * kQ4Bytes;
            const int g = (k0 / 64) & 3;
            uint4 hd = *reinterpret_cast<const uint4*>(sb);
            uint4 qv = *reinterpret_cast<const uint4*>(sb + 16 + 32 * g + 16 * h);
            float d = half_bits_to_float(hd.x);
            float dmin = half_bits_to_float(hd.x >> 16);
            Q4KScales sc = q4k_unpack(hd.y, hd.z, hd.w);
            uint32_t sc0, m0, sc1, m1;
            q4k_sub(sc, 2 * g, sc0, m0);
            q4k_sub(sc, 2 * g + 1, sc1, m1);
            const float a0 = d * (float)sc0, b0 = dmin * (float)m0;
            const float a1 = d * (float)sc1, b1 = dmin * (float)m1;
            const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t lo = qw[i] & 0x0F0F0F0Fu;
                uint32_t hi = (qw[i] >> 4) & 0x0F0F0F0Fu;
                o[2 * i] = pack_bf16x2(a0 * ubyte_f(lo, 0) - b0, a0 * ubyte_f(lo, 1) - b0);
                o[2 * i + 1] = pack_bf16x2(a0 * ubyte_f(lo, 2) - b0, a0 * ubyte_f(lo, 3) - b0);
                o[8 + 2 * i] = pack_bf16x2(a1 * ubyte_f(hi, 0) - b1, a1 * ubyte_f(hi, 1) - b1);
                o[8 + 2 * i + 1] = pack_bf16x2(a1 * ubyte_f(hi, 2) - b1, a1 * ubyte_f(hi, 3) - b1);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] = 0;
        }
        uint4* lo4 = reinterpret_cast<uint4*>(dst + 16 * h);
        uint4* hi4 = reinterpret_cast<uint4*>(dst + 32 + 16 * h);
        lo4[0] = make_uint4(o[0], o[1], o[2], o[3]);
        lo4[1] = make_uint4(o[4], o[5], o[6], o[7]);
        hi4[0] = make_uint4(o[8], o[9], o[10], o[11]);
        hi4[1] = make_uint4(o[12], o[13], o[14], o[15]);
    }
}

template <int FMT, int NT>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ w, int64_t n,
                                                   int64_t k, int64_t rb,
                                                   const uint16_t* __restrict__ abf, int64_t kp,
                                                   int64_t m, float* __restrict__ c, int64_t ldc) {
    constexpr int BN = 16 * NT;
    __shared__ __align__(16) uint16_t As[kBM * kLdsRow];
    __shared__ __align__(16) uint16_t Ws[BN * kLdsRow];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kBM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;

    f32x4 acc[2][NT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = (int)(kp / kBK);
    for (int ks = 0; ks < nsteps; ++ks) {
        const int k0 = ks * kBK;
        // A tile: 128 rows x 64 bf16 = 1024 16-byte pieces
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int p = tid + 256 * i;
            int row = p >> 3;
            int col = (p & 7) * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m0 + row < m) v = *reinterpret_cast<const uint4*>(abf + (m0 + row) * kp + k0 + col);
            *reinterpret_cast<uint4*>(As + row * kLdsRow + col) = v;
        }
        // W tile: BN rows x 64 weights, two threads per row
        for (int p = tid; p < 2 * BN; p += 256) {
            int nn = p >> 1;
            int h = p & 1;
            decode_w32<FMT>(w, n0 + nn, n0 + nn < n, rb, k, k0, h, Ws + nn * kLdsRow);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            bf16x8 af[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const uint16_t* src = As + (32 * wv + 16 * mi + (lane & 15)) * kLdsRow + kk + 8 * (lane >> 4);
                af[mi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src));
            }
#pragma unroll
            for (int nj = 0; nj < NT; ++nj) {
                const uint16_t* src = Ws + (16 * nj + (lane & 15)) * kLdsRow + kk + 8 * (lane >> 4);
                bf16x8 bfr = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src));
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr, acc[mi][nj], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    // D[i][j]: lane holds rows 4*(lane/16) + r, column lane%16
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < NT; ++nj) {
            const int64_t col = n0 + 16 * nj + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 32 * wv + 16 * mi + 4 * (lane >> 4) + r;
                if (row < m && col < n) c[row * ldc + col] = acc[mi][nj][r];
            }
        }
}

}  // namespace

size_t gemm_workspace_bytes(int type, int64_t m, int64_t n, int64_t k) {
    (void)type;
    (void)n;
    return (size_t)m * (size_t)kpad(k) * 2 + 256;
}

hipError_t launch_gemm(int type, const uint8_t* w, int64_t n, int64_t k, const float* a,
                       int64_t lda, int64_t m, float* c, int64_t ldc, void* ws, hipStream_t s) {
    const int64_t kp = kpad(k);
    uint16_t* abf = static_cast<uint16_t*>(ws);
    const int64_t total = m * (kp / 4);
    hipLaunchKernelGGL(prep_bf16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a,
                       lda, m, k, kp, abf);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t rb = row_bytes(type, k);
    constexpr int NT = 8;
    dim3 grid((unsigned)((n + 16 * NT - 1) / (16 * NT)), (unsigned)((m + kBM - 1) / kBM));
    if (type == kQ4_K)
        hipLaunchKernelGGL((gemm_kernel<kQ4_K, NT>), grid, dim3(256), 0, s, w, n, k, rb, abf, kp, m,
                           c, ldc);
    else
        hipLaunchKernelGGL((gemm_kernel<kQ8_0, NT>), grid, dim3(256), 0, s, w, n, k, rb, abf, kp, m,
                           c, ldc);
    return hipGetLastError();
}

}  // namespace ggq
