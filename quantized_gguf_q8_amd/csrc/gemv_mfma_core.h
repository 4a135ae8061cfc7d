// gemv_mfma_core.h -- matrix-core building blocks of the batched decode GEMV,
// shared by quant_gemv (batch 2..16) and the routed-expert stages.
//
// Same product as quant_gemv (Phobos README, "Inference"): y[b][r] = sum_c w[r][c] x[b][c],
// fp32-accurate, with one MFMA serving up to 8 activation rows and the vector
// units only converting the weights.
//
// Exactness of the operands:
//  * Activations: each row b is scaled by a power of two 2^S_b (max |x| lands in
//    [2^14, 2^15)) and split as x' = hi + lo with hi = fp16(x'), lo = fp16(x' - hi);
//    hi + lo carries 22 significant bits.  A pre-kernel writes these as MFMA
//    A-operand fragments (rows i = 2*b + {0: hi, 1: lo}) once per call.
//  * Q8_0 weights: q (int8) is exact in fp16.  Bytes become fp16 by the classic
//    exponent trick: (q ^ 0x80) in the low byte under exponent byte 0x64 is
//    fp16(1024 + q + 128); subtracting 1152 gives q exactly.  Each 32-weight block
//    is one v_mfma_f32_16x16x32_f16 whose 16x16 result is scaled by its row's d.
//  * Q4_K weights: sc*q <= 945 is exact in fp16, made as fma(1024 + q, sc, -1024*sc).
//    A super-block's eight sub-blocks therefore accumulate inside the MFMA and are
//    scaled once by d.  The min term -dmin * sum_j m_j * sum_{c in j} x_c is a
//    second, 16x16x16 MFMA per super-block: m_j (6-bit, exact) against the
//    per-sub-block activation sums (scaled by 2^(S_b - 5) so they fit fp16).
//  * Products of fp16 values are exact in fp32; sums accumulate in fp32.
//
#pragma once

#include "gemv_core.h"

namespace ggq {

namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kMaxJobs = 16;

__host__ __device__ constexpr int64_t al256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Workspace layout per job (byte offsets from the job's base).
struct XfLayout {
    int64_t frag;   // [MT][K/32][64 lanes][8 fp16]
    int64_t mins;   // Q4_K: [MT][K/256][64 lanes][4 fp16]
    int64_t inv;    // [MT*8] fp32: 2^-S_b
    int64_t ctrl;   // 256 bytes: the work counter of a grouped launch (first job's region)
    int64_t bytes;
};

__host__ __device__ inline XfLayout xf_layout(int type, int64_t k, int mt) {
    XfLayout L;
    L.frag = 0;
    L.mins = al256((int64_t)mt * (k / 32) * 1024);
    const int64_t mb = type == kQ4_K ? (int64_t)mt * (k / 256) * 512 : 0;
    L.inv = L.mins + al256(mb);
    L.ctrl = L.inv + al256((int64_t)mt * 8 * 4);    // 2^-S per padded row
    L.bytes = L.ctrl + 256;
    return L;
}

// A job's work items are its row tiles, each whole or cut into nsplit K parts
// of cpp chunks.  Two parts are added into y, which the pre-kernel zeroes: two
// additions onto an exact zero give the same bits in either order.  More parts
// write partial sums to `part` ([nsplit][batch][n] floats), which a second
// kernel adds in part order.
constexpr int kMaxParts = 16;

struct MJob {
    const uint8_t* w;
    const float* x;
    float* y;
    uint8_t* xf;      // this job's workspace region
    float* part;      // partial sums region (kMaxParts * batch * n floats), or null
    int64_t n, ldx, ldy, rb;
    int32_t k, nchunk, item0, tiles, nsplit, cpp;
};

struct MJobs {
    MJob j[kMaxJobs];
    int32_t* ctr;     // work counter (zeroed by the pre-kernel), or null
    int32_t count;
    int32_t total_items;
    int32_t batch;    // activation rows (partial-sum plane height)
};

// ------------------------------------------------------------------ prep ----
// One workgroup per (job, padded batch row b).  Rows b >= batch write zeros so the
// padded MFMA rows contribute nothing.
// blockIdx.y splits K into slices of kXfragSlice blocks (one slice up to K =
// 16384).  A thread holds its pieces of the slice (8 floats each) in registers
// from the single read that also gives the maximum; a row longer than one
// slice is scanned once more for its maximum, so slices need no exchange.
constexpr int kXfragPer = 8;                      // pieces per thread
constexpr int kXfragSlice = 256 * kXfragPer / 4;  // 32-weight blocks per slice

// One workgroup's share: bx = (job, padded row), slice `slice` of `nslices`.
template <int FMT>
__device__ __forceinline__ void xfrag_block(const MJobs& jobs, int batch, int mt, int bx, int slice,
                                            int nslices) {
    const int job = bx / (mt * 8);
    const int b = bx % (mt * 8);
    const MJob& jb = jobs.j[job];
    const int k = jb.k;
    const XfLayout L = xf_layout(FMT, k, mt);
    const int tid = threadIdx.x;
    const bool live = b < batch;
    const float* xb = jb.x + (int64_t)(live ? b : 0) * jb.ldx;

    // Outputs of split jobs are sums of two halves: start them at zero.  The
    // slices of this (job, row) share the N rows between them.
    if (jb.nsplit == 2 && live) {
        const int64_t r0 = jb.n * slice / nslices, r1 = jb.n * (slice + 1) / nslices;
        float* yb = jb.y + (int64_t)b * jb.ldy;
        for (int64_t r = r0 + tid; r < r1; r += 256) yb[r] = 0.f;
    }
    if (jobs.ctr && bx == 0 && slice == 0 && tid == 0) *jobs.ctr = 0;

    const int nblk = k / 32;
    const int q0 = slice * kXfragSlice * 4;             // first piece of the slice
    const int q1 = min(nblk, (slice + 1) * kXfragSlice) * 4;
    if (q0 >= nblk * 4) return;                          // this job's row is shorter
    // piece q = (block q/4, octet q%4): 8 consecutive floats
    float xv[kXfragPer][8];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < kXfragPer; ++i) {
        const int q = q0 + tid + 256 * i;
#pragma unroll
        for (int c = 0; c < 8; ++c) xv[i][c] = 0.f;
        if (live && q < q1) {
            const float4 a = *reinterpret_cast<const float4*>(xb + q * 8);
            const float4 a2 = *reinterpret_cast<const float4*>(xb + q * 8 + 4);
            xv[i][0] = a.x; xv[i][1] = a.y; xv[i][2] = a.z; xv[i][3] = a.w;
            xv[i][4] = a2.x; xv[i][5] = a2.y; xv[i][6] = a2.z; xv[i][7] = a2.w;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(xv[i][c]));
    }
    if (live && nslices > 1) {
        // the rest of the row, for the row's maximum
        const float4* x4 = reinterpret_cast<const float4*>(xb);
        for (int c = tid; c < k / 4; c += 256) {
            if (c >= q0 * 2 && c < q1 * 2) continue;
            const float4 v = x4[c];
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    }

    // max |x_b| -> scale 2^S with max * 2^S in [2^14, 2^15)
    __shared__ float red[4];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    float sc = 1.f, inv = 1.f;
    if (live && m > 0.f && m <= 3.4e38f) {
        frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1)
        sc = ldexpf(1.f, 15 - e);
        inv = ldexpf(1.f, e - 15);
    }
    const int t = b / 8;          // M tile
    const int bb = b % 8;         // row pair within the tile
    if (tid == 0 && slice == 0) reinterpret_cast<float*>(jb.xf + L.inv)[b] = live ? inv : 1.f;

    // A-operand fragments of v_mfma_f32_16x16x32_f16: lane l = i + 16*h holds
    // A[i][8h .. 8h+7]; rows i = 2*bb (hi) and 2*bb + 1 (lo).
    _Float16* frag = reinterpret_cast<_Float16*>(jb.xf + L.frag);
    _Float16* mins = reinterpret_cast<_Float16*>(jb.xf + L.mins);
    const int nsb = k / 256;
    const float sc5 = sc * (1.f / 32.f);
#pragma unroll
    for (int i = 0; i < kXfragPer; ++i) {
        const int q = q0 + tid + 256 * i;
        // a block's four pieces (four consecutive lanes) are all in or all out,
        // which is all the sub-block sums below need from their shuffles
        if (q >= q1) continue;
        const int blk = q >> 2;
        const int h = q & 3;
        f16x8 hi, lo;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float v = xv[i][c] * sc;
            const _Float16 vh = (_Float16)v;
            hi[c] = vh;
            lo[c] = (_Float16)(v - (float)vh);
        }
        _Float16* base = frag + ((int64_t)(t * nblk + blk) * 64) * 8;
        *reinterpret_cast<f16x8*>(base + (2 * bb + 16 * h) * 8) = hi;
        *reinterpret_cast<f16x8*>(base + (2 * bb + 1 + 16 * h) * 8) = lo;
        if constexpr (FMT == kQ4_K) {
            // A operand of v_mfma_f32_16x16x16_f16: lane l = i + 16*hq holds
            // A[i][4hq .. 4hq+3]; k = sub-block index 0..7 (hq 0, 1); hq 2, 3
            // are zero.  Sub-block j of super-block sb is block 8*sb + j: its
            // four pieces sit in four consecutive lanes.
            float sblk = ((xv[i][0] + xv[i][1]) + (xv[i][2] + xv[i][3])) +
                         ((xv[i][4] + xv[i][5]) + (xv[i][6] + xv[i][7]));
            sblk += __shfl_xor(sblk, 1, 64);
            sblk += __shfl_xor(sblk, 2, 64);
            const int sb = blk >> 3;
            const int j = blk & 7;
            _Float16* mb = mins + ((int64_t)(t * nsb + sb) * 64) * 4;
            if (h == 0) {
                const float v = sblk * sc5;
                const _Float16 vh = (_Float16)v;
                const int hq = j >> 2, jj = j & 3;
                mb[(2 * bb + 16 * hq) * 4 + jj] = vh;
                mb[(2 * bb + 1 + 16 * hq) * 4 + jj] = (_Float16)(v - (float)vh);
            } else if (h == 1 && j == 0) {
#pragma unroll
                for (int hq = 2; hq < 4; ++hq) {
                    *reinterpret_cast<f16x4*>(mb + (2 * bb + 16 * hq) * 4) = f16x4{0, 0, 0, 0};
                    *reinterpret_cast<f16x4*>(mb + (2 * bb + 1 + 16 * hq) * 4) = f16x4{0, 0, 0, 0};
                }
            }
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void xfrag_kernel(const MJobs jobs, int batch, int mt) {
    xfrag_block<FMT>(jobs, batch, mt, blockIdx.x, blockIdx.y, gridDim.y);
}

// ------------------------------------------------------------- helpers ----
// Four int8 in v -> two fp16x2 holding exactly those integers.
__device__ __forceinline__ void q8x4_to_f16(uint32_t v, uint32_t& o0, uint32_t& o1) {
    const uint32_t u = v ^ 0x80808080u;
    const uint32_t e = 0x64646464u;
    f16x2 a = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, u, 0x04010400u));
    f16x2 b = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, u, 0x04030402u));
    const f16x2 off = {(_Float16)1152.f, (_Float16)1152.f};
    o0 = __builtin_bit_cast(uint32_t, a - off);
    o1 = __builtin_bit_cast(uint32_t, b - off);
}

// Four nibble-valued bytes in v (each 0..15) -> two fp16x2 holding sc*q exactly.
__device__ __forceinline__ void q4x4_to_f16(uint32_t v, f16x2 sc2, f16x2 msc2, uint32_t& o0,
                                            uint32_t& o1) {
    const uint32_t e = 0x64646464u;
    f16x2 a = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, v, 0x04010400u));
    f16x2 b = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, v, 0x04030402u));
    o0 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(a, sc2, msc2));
    o1 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(b, sc2, msc2));
}

// KCQ4: weights per chunk for Q4_K, 512 (two super-blocks) or 256; Q8_0 chunks
// are 256 weights.
template <int FMT, int MT, int WM, int KCQ4 = 512>
struct MCfg {
    static_assert(KCQ4 == 512 || KCQ4 == 256, "Q4_K chunk");
    static constexpr int WK = 4 / WM;
    static constexpr int RWG = 16 * WM;                         // rows per workgroup
    static constexpr int KC = FMT == kQ8_0 ? 256 : KCQ4;        // weights per chunk
    static constexpr int CRB = FMT == kQ8_0 ? 272 : KC / 256 * 144;   // bytes per row chunk
    // LDS row stride: 68 dwords (Q8_0) / 76 or 44 dwords (Q4_K) put the 16 rows a
    // wave reads at distinct multiples of 4 banks, so 64 lanes x 2 dwords spread
    // evenly.
    static constexpr int RS = FMT == kQ8_0 ? CRB : CRB + (KC == 512 ? 16 : 32);
    static constexpr int NBLK = KC / 32;                        // 32-wide steps per chunk
    static constexpr int NSB = FMT == kQ4_K ? KC / 256 : 0;
    static constexpr int kW = RWG * RS;
    static constexpr int kFrag = MT * NBLK * 1024;
    static constexpr int kMins = MT * NSB * 512;
    static constexpr int kBuf = kW + kFrag + kMins;
    static constexpr int kRed = WK > 1 ? WK * WM * 64 * MT * 4 * 4 : 0;
    static constexpr int kLds = 2 * kBuf + kRed;
    static constexpr int WPIECES = RWG * CRB / 16;
    static constexpr int WP = (WPIECES + 255) / 256;
    static constexpr int FPIECES = (kFrag + kMins) / 16;
    static constexpr int FP = (FPIECES + 255) / 256;
};

// The products of one K chunk staged in LDS (weights of this wave's rows,
// activation fragments) into acc: Q8_0 per 32-weight block, Q4_K per
// super-block with its min term.  k0 is the chunk's first column, kval the
// matrix's K.
template <int FMT, int MT, int WM, int KCQ4 = 512>
__device__ __forceinline__ void mfma_chunk(const uint8_t* lds, int k0, int kval, int lane, int wm,
                                           int wk, int j, int h, f32x4 (&acc)[MT]) {
    using C = MCfg<FMT, MT, WM, KCQ4>;
    constexpr int WK = C::WK;
    const uint8_t* base = lds;
    const uint8_t* wrow = base + (16 * wm + j) * C::RS;
    const uint8_t* frag = base + C::kW;
    if constexpr (FMT == kQ8_0) {
        // K is a multiple of the chunk here, so every block is present.
        // Blocks are taken in pairs (68 bytes, dword aligned): the even
        // block's quants start 2 bytes into a dword and are realigned, the
        // odd block's are aligned; its scale is the high half of dword 8.
        constexpr int NPW = C::NBLK / WK;   // blocks per wave: pairs wk, wk+WK, ...
        static_assert(NPW % 2 == 0, "blocks per wave come in pairs");
        f16x8 bop[NPW];
        float dq[NPW];
        const uint32_t* rowd = reinterpret_cast<const uint32_t*>(wrow);
#pragma unroll
        for (int i = 0; i < NPW; i += 2) {
            const int pr = wk + WK * (i >> 1);   // pair index in the chunk
            const uint32_t* pd = rowd + 17 * pr;
            const uint32_t e0 = pd[2 * h], e1 = pd[2 * h + 1], e2 = pd[2 * h + 2];
            const uint32_t o0 = pd[9 + 2 * h], o1 = pd[10 + 2 * h];
            dq[i] = half_bits_to_float(pd[0]);
            dq[i + 1] = half_bits_to_float(pd[8] >> 16);
            uint32_t b4[4];
            q8x4_to_f16(__builtin_amdgcn_alignbyte(e1, e0, 2), b4[0], b4[1]);
            q8x4_to_f16(__builtin_amdgcn_alignbyte(e2, e1, 2), b4[2], b4[3]);
            bop[i] = __builtin_bit_cast(f16x8, make_uint4(b4[0], b4[1], b4[2], b4[3]));
            q8x4_to_f16(o0, b4[0], b4[1]);
            q8x4_to_f16(o1, b4[2], b4[3]);
            bop[i + 1] = __builtin_bit_cast(f16x8, make_uint4(b4[0], b4[1], b4[2], b4[3]));
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            f32x4 dv[NPW];
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
                const int bi = 2 * (wk + WK * (i >> 1)) + (i & 1);
                const f16x8 aop = *reinterpret_cast<const f16x8*>(
                    frag + (t * C::NBLK + bi) * 1024 + lane * 16);
                dv[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[i],
                                                              f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < NPW; ++i) acc[t] += dq[i] * dv[i];
        }
    } else {
#pragma unroll
        for (int si = wk; si < C::NSB; si += WK) {
            if (k0 + 256 * si < kval) {
                const uint8_t* sb = wrow + si * kQ4Bytes;
                const uint4 hd = *reinterpret_cast<const uint4*>(sb);
                const float d = half_bits_to_float(hd.x);
                const float dmin = half_bits_to_float(hd.x >> 16);
                const Q4KScales scl = q4k_unpack(hd.y, hd.z, hd.w);
                f32x4 dsb[MT], dmn[MT];
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    dsb[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                    dmn[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint2 qv = *reinterpret_cast<const uint2*>(sb + 16 + 32 * c + 8 * h);
#pragma unroll
                    for (int hi = 0; hi < 2; ++hi) {
                        const int sub = 2 * c + hi;
                        uint32_t scj, mj;
                        q4k_sub(scl, sub, scj, mj);
                        const _Float16 sch = (_Float16)(float)scj;
                        const _Float16 msch = (_Float16)(-1024.f * (float)scj);
                        const f16x2 sc2 = {sch, sch};
                        const f16x2 msc2 = {msch, msch};
                        const uint32_t n0 = hi ? (qv.x >> 4) & 0x0F0F0F0Fu : qv.x & 0x0F0F0F0Fu;
                        const uint32_t n1 = hi ? (qv.y >> 4) & 0x0F0F0F0Fu : qv.y & 0x0F0F0F0Fu;
                        uint32_t b4[4];
                        q4x4_to_f16(n0, sc2, msc2, b4[0], b4[1]);
                        q4x4_to_f16(n1, sc2, msc2, b4[2], b4[3]);
                        const f16x8 bop =
                            __builtin_bit_cast(f16x8, make_uint4(b4[0], b4[1], b4[2], b4[3]));
                        const int step = si * 8 + sub;
#pragma unroll
                        for (int t = 0; t < MT; ++t) {
                            const f16x8 aop = *reinterpret_cast<const f16x8*>(
                                frag + (t * C::NBLK + step) * 1024 + lane * 16);
                            dsb[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, dsb[t], 0, 0, 0);
                        }
                    }
                }
                // min term: B[k][col] = m_k of this row for k < 8, zero above
                uint32_t mv = h == 0 ? scl.mnl : scl.mnh;
                uint32_t m0 = 0, m1 = 0;
                if (h < 2) {
                    const uint32_t e = 0x64646464u;
                    const f16x2 off = {(_Float16)1024.f, (_Float16)1024.f};
                    m0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, mv, 0x04010400u)) - off);
                    m1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(e, mv, 0x04030402u)) - off);
                }
                const f16x4 mop = __builtin_bit_cast(f16x4, make_uint2(m0, m1));
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const f16x4 xop = *reinterpret_cast<const f16x4*>(
                        frag + C::kFrag + (t * C::NSB + si) * 512 + lane * 8);
                    dmn[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(xop, mop, dmn[t], 0, 0, 0);
                    acc[t] += d * dsb[t] - (32.f * dmin) * dmn[t];
                }
            }
        }
    }
}

}  // namespace

}  // namespace ggq
