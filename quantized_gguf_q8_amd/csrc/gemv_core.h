// gemv_core.h -- the decode-GEMV building blocks shared by quant_gemv's
// streaming kernel and the routed-expert kernels.
//
// Per-token products over GGUF weights (Phobos README, "Inference"); the routed
// experts reuse them with gathered activations (README opening paragraph).
//
// Thread layout: a workgroup of 256 threads covers ROWS rows, each row split
// into SL = 256/ROWS K-slices (slice fastest, so a row's slices are lanes of one
// wave).  A thread's unit is 64 consecutive weights of its row -- two Q8_0
// blocks (68 bytes) or a 64-weight quarter of a Q4_K super-block (its 16-byte
// header + 32 quant bytes) -- and K is walked in chunks of KC = 64*SL weights.
// A chunk of a row is contiguous in memory, so the row chunks of a tile are
// copied to LDS with coalesced 16-byte loads (34-byte Q8_0 blocks never need
// unaligned global loads); the activation chunk is staged beside it, padded per
// slice so the slices a wave reads land in distinct LDS bank groups.
// Q4_K is evaluated per 32-weight sub-block j in the factored form
//     d*sc_j * sum q_c x_c  -  dmin*m_j * sum x_c,
// with sum x_c formed once per chunk while the activations are staged.
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

// Rows per workgroup for a given batch cap and K: the smallest of 8/16/32/64
// that keeps the activation chunk within ~34 KB of LDS (ROWS >= 2*NB) and the
// chunk no wider than K.
__host__ inline int gemv_rows_for(int nb, int64_t k) {
    int rows = 8;
    while (rows < 64 && (rows < 2 * nb || (16384 / rows) > k)) rows *= 2;
    return rows;
}

}  // namespace ggq
