// gemv_core.h -- the workgroup-level decode GEMV shared by quant_gemv and the
// routed-expert kernels.
//
// Computes, for ROWS consecutive rows r of NMAT quantized matrices (same shape,
// same activations) and up to NB activation rows b:
//     v[m][b][r] = sum_c w_m[r][c] * x_b[c]
// and hands each finished value to an epilogue functor.  Phobos README,
// "Inference": the per-token product over GGUF weights; the routed experts reuse
// it with gathered activations (README opening paragraph).
//
// Decomposition (256 threads, wave64):
//  * The 256 threads are SL = 256/ROWS K-slices of each row (slice fastest);
//    a thread's unit is 64 consecutive weights: two Q8_0 blocks (68 bytes) or one
//    64-weight quarter of a Q4_K super-block (the 16-byte header + 32 quant bytes).
//  * K is walked in chunks of KC = 64*SL weights.  A chunk of a row is contiguous
//    in memory; the workgroup copies the chunk of all its rows to LDS with 16-byte
//    loads, coalesced along each row, so the 34-byte Q8_0 blocks never need
//    unaligned global loads.  The activation chunk is staged beside it, padded per
//    slice so the 16 slices a wave reads land in distinct LDS bank groups.
//  * A thread decodes its unit once into registers and applies it to every
//    activation row: one read of the weights serves the whole batch.
//  * The SL partials of a row are summed through LDS in a fixed order, so the
//    result does not depend on timing.
//  * Q4_K is evaluated per 32-weight sub-block j in the factored form
//        d*sc_j * sum q_c x_c  -  dmin*m_j * sum x_c,
//    with sum x_c computed once per chunk while the activations are staged.
#pragma once

#include "ggq_device.h"

namespace ggq {

template <int FMT>
struct UnitBytes {
    static constexpr int value = FMT == kQ8_0 ? 68 : 36;  // bytes per 64 weights
};

template <int FMT, int NB, int ROWS, int NMAT>
struct GemvCfg {
    static constexpr int SL = 256 / ROWS;                 // K-slices per row
    static constexpr int KC = SL * 64;                    // weights per row per chunk
    static constexpr int CRB = SL * UnitBytes<FMT>::value;  // chunk bytes per row
    static constexpr int WRS = CRB + 16;                  // LDS row stride (bytes)
    static constexpr int XSS = 68;                        // floats per slice (64 + pad)
    static constexpr int XBS = SL * XSS;                  // floats per activation row
    static constexpr int kWBytes = NMAT * ROWS * WRS;
    static constexpr int kXBytes = NB * XBS * 4;
    static constexpr int kSumBytes = FMT == kQ4_K ? NB * SL * 2 * 4 : 0;
    static constexpr int kRedBytes = NMAT * NB * ROWS * (SL + 1) * 4;
    static constexpr int kMain = kWBytes + kXBytes + kSumBytes;
    static constexpr int kLds = kMain > kRedBytes ? kMain : kRedBytes;
    static_assert(SL % 4 == 0 && SL <= 64, "slice count");
    static_assert(CRB % 16 == 0, "chunk rows must be whole 16-byte pieces");
    static_assert((NB * KC / 4) % 64 == 0, "activation staging must use whole waves");
};

// Decode this thread's 64-weight unit from LDS into two 32-float halves with
// their scales (sa) and, for Q4_K, min terms (mb).
template <int FMT>
__device__ __forceinline__ void decode_unit(const uint8_t* row, int s, float (&f0)[32],
                                            float (&f1)[32], float& sa0, float& sa1, float& mb0,
                                            float& mb1) {
    if constexpr (FMT == kQ8_0) {
        const uint32_t* u = reinterpret_cast<const uint32_t*>(row + s * 68);
        uint32_t dw[17];
#pragma unroll
        for (int i = 0; i < 17; ++i) dw[i] = u[i];
        sa0 = half_bits_to_float(dw[0]);
        sa1 = half_bits_to_float(dw[8] >> 16);
        mb0 = mb1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // block 0's quants start at byte 2: realign two dwords
            uint32_t q0 = __builtin_amdgcn_alignbyte(dw[i + 1], dw[i], 2);
            uint32_t q1 = dw[9 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f0[4 * i + j] = sbyte_f(q0, j);
                f1[4 * i + j] = sbyte_f(q1, j);
            }
        }
    } else {
        const uint8_t* sb = row + (s >> 2) * kQ4Bytes;
        const int g = s & 3;  // 64-weight group: sub-blocks 2g (low nibbles), 2g+1 (high)
        uint4 hd = *reinterpret_cast<const uint4*>(sb);
        float d = half_bits_to_float(hd.x);
        float dmin = half_bits_to_float(hd.x >> 16);
        Q4KScales sc = q4k_unpack(hd.y, hd.z, hd.w);
        uint32_t sc0, m0, sc1, m1;
        q4k_sub(sc, 2 * g, sc0, m0);
        q4k_sub(sc, 2 * g + 1, sc1, m1);
        sa0 = d * (float)sc0;
        sa1 = d * (float)sc1;
        mb0 = dmin * (float)m0;
        mb1 = dmin * (float)m1;
        const uint32_t* q = reinterpret_cast<const uint32_t*>(sb + 16 + 32 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t v = q[i];
            uint32_t lo = v & 0x0F0F0F0Fu;
            uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f0[4 * i + j] = ubyte_f(lo, j);
                f1[4 * i + j] = ubyte_f(hi, j);
            }
        }
    }
}

// One 32-weight half of the unit decode_unit covers (half 0: the first Q8_0
// block / the low nibbles; half 1: the second block / the high nibbles), for
// callers that keep fewer registers live.
template <int FMT>
__device__ __forceinline__ void decode_half(const uint8_t* row, int s, int half, float (&f)[32],
                                            float& sa, float& mb) {
    if constexpr (FMT == kQ8_0) {
        const uint32_t* u = reinterpret_cast<const uint32_t*>(row + s * 68);
        if (half == 0) {
            uint32_t dw[9];
#pragma unroll
            for (int i = 0; i < 9; ++i) dw[i] = u[i];
            sa = half_bits_to_float(dw[0]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t q = __builtin_amdgcn_alignbyte(dw[i + 1], dw[i], 2);
#pragma unroll
                for (int j = 0; j < 4; ++j) f[4 * i + j] = sbyte_f(q, j);
            }
        } else {
            sa = half_bits_to_float(u[8] >> 16);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t q = u[9 + i];
#pragma unroll
                for (int j = 0; j < 4; ++j) f[4 * i + j] = sbyte_f(q, j);
            }
        }
        mb = 0.f;
    } else {
        const uint8_t* sb = row + (s >> 2) * kQ4Bytes;
        const int g = s & 3;
        const uint4 hd = *reinterpret_cast<const uint4*>(sb);
        const Q4KScales sc = q4k_unpack(hd.y, hd.z, hd.w);
        uint32_t scj, mj;
        q4k_sub(sc, 2 * g + half, scj, mj);
        sa = half_bits_to_float(hd.x) * (float)scj;
        mb = half_bits_to_float(hd.x >> 16) * (float)mj;
        const uint32_t* q = reinterpret_cast<const uint32_t*>(sb + 16 + 32 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = half ? (q[i] >> 4) & 0x0F0F0F0Fu : q[i] & 0x0F0F0F0Fu;
#pragma unroll
            for (int j = 0; j < 4; ++j) f[4 * i + j] = ubyte_f(v, j);
        }
    }
}

// xrow[b]: activation row b (valid for b < batch).  w[m]: base of matrix m.
// epi(b, r, v): v[m] is the finished product of row r with activation row b.
template <int FMT, int NB, int ROWS, int NMAT, class Epi>
__device__ __forceinline__ void gemv_tile(uint8_t* lds, const uint8_t* const (&w)[NMAT], int64_t n,
                                          int k, int64_t rbytes, const float* const (&xrow)[NB],
                                          int batch, int64_t r0, Epi& epi) {
    using C = GemvCfg<FMT, NB, ROWS, NMAT>;
    constexpr int SL = C::SL;
    constexpr int KC = C::KC;
    uint8_t* lw = lds;
    float* lx = reinterpret_cast<float*>(lds + C::kWBytes);
    float* lsum = reinterpret_cast<float*>(lds + C::kWBytes + C::kXBytes);

    const int tid = threadIdx.x;
    const int s = tid % SL;
    const int rl = tid / SL;
    const bool row_ok = r0 + rl < n;

    float acc[NMAT][NB];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[m][b] = 0.f;

    const int nchunks = (k + KC - 1) / KC;
    for (int c = 0; c < nchunks; ++c) {
        const int k0 = c * KC;
        {   // weights: NMAT x ROWS rows x CRB bytes as 16-byte pieces
            constexpr int PPR = C::CRB / 16;
            const int64_t cb0 = (int64_t)c * C::CRB;
            for (int p = tid; p < NMAT * ROWS * PPR; p += 256) {
                int m = p / (ROWS * PPR);
                int pr = (p / PPR) % ROWS;
                int off = (p % PPR) * 16;
                if (r0 + pr < n && cb0 + off < rbytes) {
                    const uint4* src =
                        reinterpret_cast<const uint4*>(w[m] + (r0 + pr) * rbytes + cb0 + off);
                    *reinterpret_cast<uint4*>(lw + (m * ROWS + pr) * C::WRS + off) = *src;
                }
            }
        }
        {   // activations [NB][KC] (+ per-32 sums for Q4_K)
            constexpr int P4 = KC / 4;
            for (int p = tid; p < NB * P4; p += 256) {
                int b = p / P4;
                int pos = (p % P4) * 4;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (b < batch && k0 + pos < k)
                    v = *reinterpret_cast<const float4*>(xrow[b] + k0 + pos);
                *reinterpret_cast<float4*>(lx + b * C::XBS + (pos >> 6) * C::XSS + (pos & 63)) = v;
                if constexpr (FMT == kQ4_K) {
                    // 8 consecutive lanes hold one 32-weight run
                    float t = (v.x + v.y) + (v.z + v.w);
                    t += __shfl_xor(t, 1, 64);
                    t += __shfl_xor(t, 2, 64);
                    t += __shfl_xor(t, 4, 64);
                    if ((p & 7) == 0) lsum[(b * SL + (pos >> 6)) * 2 + ((pos >> 5) & 1)] = t;
                }
            }
        }
        __syncthreads();

        if (row_ok && k0 + s * 64 < k) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                float f0[32], f1[32];
                float sa0, sa1, mb0, mb1;
                decode_unit<FMT>(lw + (m * ROWS + rl) * C::WRS, s, f0, f1, sa0, sa1, mb0, mb1);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < batch) {
                        const float4* xv =
                            reinterpret_cast<const float4*>(lx + b * C::XBS + s * C::XSS);
                        float p0[4] = {0.f, 0.f, 0.f, 0.f}, p1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            float4 a = xv[i];
                            float4 e = xv[8 + i];
                            p0[i & 3] += f0[4 * i] * a.x + f0[4 * i + 1] * a.y +
                                         f0[4 * i + 2] * a.z + f0[4 * i + 3] * a.w;
                            p1[i & 3] += f1[4 * i] * e.x + f1[4 * i + 1] * e.y +
                                         f1[4 * i + 2] * e.z + f1[4 * i + 3] * e.w;
                        }
                        float s0 = (p0[0] + p0[1]) + (p0[2] + p0[3]);
                        float s1 = (p1[0] + p1[1]) + (p1[2] + p1[3]);
                        float t = sa0 * s0 + sa1 * s1;
                        if constexpr (FMT == kQ4_K) {
                            const float* xs = lsum + (b * SL + s) * 2;
                            t -= mb0 * xs[0] + mb1 * xs[1];
                        }
                        acc[m][b] += t;
                    }
                }
            }
        }
        __syncthreads();
    }

    // slice partials -> LDS -> fixed-order sums
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int b = 0; b < NB; ++b) red[((m * NB + b) * ROWS + rl) * (SL + 1) + s] = acc[m][b];
    __syncthreads();
    for (int o = tid; o < NB * ROWS; o += 256) {
        int b = o / ROWS;
        int r = o % ROWS;
        if (b < batch && r0 + r < n) {
            float v[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const float* q = red + ((m * NB + b) * ROWS + r) * (SL + 1);
                float pr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < SL; ++i) pr[i & 3] += q[i];
                v[m] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
            }
            epi(b, r0 + r, v);
        }
    }
}

// Rows per workgroup for a given batch cap and K: the smallest of 8/16/32/64
// that keeps the activation chunk within ~34 KB of LDS (ROWS >= 2*NB) and the
// chunk no wider than K.
__host__ inline int gemv_rows_for(int nb, int64_t k) {
    int rows = 8;
    while (rows < 64 && (rows < 2 * nb || (16384 / rows) > k)) rows *= 2;
    return rows;
}

}  // namespace ggq
