// gemv_ks.hip -- quant_gemv for one matrix in a single launch, batch 1..16, on
// the matrix cores (Phobos README, "Inference": the decode-time product).
//
// Where it pays: matrices of a few to a few tens of MB (a 1024 x 1024 Q8_0
// projection, the 9728 x 2560 / 2560 x 9728 Q4_K feed-forward pair).  There the
// whole product is over in a few microseconds, so every extra dependent launch
// (an activation pre-pass, a partial-sum pass) costs as much as the product
// itself, and the data must be requested all at once to keep HBM busy.
//
// Workgroup = 4 waves = one row tile of 16*T rows x four 256-column units; wave
// w takes unit w.  In order:
//  1. each lane issues the loads of all of its wave's weight bytes (straight into
//     registers, in the layout the MFMA B operand needs: lane (j, h) of a 16-row
//     tile holds row j's bytes for k-octet h), then
//  2. while they are in flight each wave splits its unit's activations into
//     exact fp16 (hi, lo) pairs in its own LDS region: each batch row b is
//     scaled by a power of two 2^S_b from the largest |x| of the wave's 256
//     columns (so the largest lands in [2^14, 2^15)), hi = fp16(x'),
//     lo = fp16(x' - hi); no other wave reads them, so no barrier is needed.
//     Q4_K launches of more workgroups than compute units split first and
//     issue the weight loads after: a compute unit returns loads in the order
//     they were issued, so activation loads issued behind a full chip's weight
//     requests wait for them (measured: 9.6 against 10.1 us for 9728 x 2560 at
//     batch 4; Q8_0 and one-round launches lose 0.3-0.6 us the same way),
//  3. the products: v_mfma_f32_16x16x32_f16, A = activation pairs (rows 2b: hi,
//     2b+1: lo), B = the decoded weights (Q8_0: q, scaled by d per 32-column
//     block; Q4_K: sc*q <= 945, exact in fp16, scaled by d per super-block, the
//     min term as one 16x16x16 MFMA of m_j against the sub-block sums of x),
//  4. each wave scales its sums by 2^-S_b (exact) and the four waves' sums are
//     added in wave order.
// Rows too few to fill the chip are cut along K: the workgroups of a row tile
// write their sums to the workspace (device-coherent stores), wait for them to
// complete, count themselves on the tile's counter (one atomic add), and the
// last one adds the parts in part order -- the same order whatever the arrival
// order, so results are deterministic.  The counters live in the workspace's
// control block, which starts at zero and which the last workgroup of each tile
// returns to zero, so repeated calls and replayed HIP graphs start clean.
#include <algorithm>

#include "gemv_mfma_core.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

constexpr int kKsWaves = 4;
constexpr int kKsUnit = 256;                  // columns per wave
constexpr int kKsCols = kKsWaves * kKsUnit;   // columns per workgroup
constexpr int kKsMaxSplitTiles = (int)(kCtrlBytes / 4);   // one counter per row tile

struct KsArgs {
    const uint8_t* w;
    const float* x;
    float* y;
    uint32_t* ctr;             // [tiles]: parts counted (control block, zero between calls)
    float* part;               // [tiles][parts][8*MT][ROWS] partial sums
    int64_t n, ldx, ldy;
    uint32_t rb;               // bytes per row
    int32_t k, nunit, tiles, parts, batch;
};

template <int FMT, int MT, int T>
struct KsCfg {
    static constexpr int ROWS = 16 * T;
    static constexpr int FRAG = 8 * MT * 1024;                 // A fragments of one unit
    static constexpr int MINS = FMT == kQ4_K ? MT * 512 : 0;   // Q4_K sub-block sums
    static constexpr int UNIT = FRAG + MINS;
    static constexpr int RED = T * MT * 64 * 8;                // one wave's (v0, v1) sums
    static_assert(RED <= UNIT, "a wave's sums fit its own fragment region");
    static constexpr int kLds = kKsWaves * UNIT;
    static constexpr int PP = 4 * MT;                          // activation pieces per lane
};

// Raw weight bytes of one 16-row tile of a unit, per lane (j, h).
template <int FMT>
struct KsRaw;
template <>
struct KsRaw<kQ4_K> {
    uint4 hd;       // d, dmin, packed scales and mins of row j's super-block
    uint4 q0, q1;   // quant bytes 32h .. 32h+31 (sub-blocks 2h: low, 2h+1: high nibbles)
};
template <>
struct KsRaw<kQ8_0> {
    // per block pair p (68 bytes): dwords 2h..2h+2 (even block's quants 8h..8h+7,
    // 2 bytes in), dwords 9+2h, 10+2h (odd block's), dword 0 (d0) and 8 (d1 high)
    uint32_t e[4][3], o[4][2], d0[4], d1[4];
};

template <int FMT, int T>
__device__ __forceinline__ void ks_load_w(const KsArgs& a, int64_t r0, int unit, bool live,
                                          int j, int h, KsRaw<FMT> (&raw)[T]) {
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (uint32_t)(a.n * a.rb));
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int64_t row = r0 + 16 * t + j;
        const bool ok = live && row < a.n;
        if constexpr (FMT == kQ4_K) {
            const uint32_t o = (uint32_t)row * a.rb + (uint32_t)unit * kQ4Bytes;
            raw[t].hd = buf_load16<false>(rw, ok ? o : kOob);
            raw[t].q0 = buf_load16<false>(rw, ok ? o + 16 + 32 * h : kOob);
            raw[t].q1 = buf_load16<false>(rw, ok ? o + 32 + 32 * h : kOob);
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t o = (uint32_t)row * a.rb + (uint32_t)unit * 272 + 68 * p;
                const auto v3 = __builtin_amdgcn_raw_buffer_load_b96(rw, ok ? o + 8 * h : kOob, 0, 0);
                const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rw, ok ? o + 36 + 8 * h : kOob, 0, 0);
                raw[t].e[p][0] = v3[0];
                raw[t].e[p][1] = v3[1];
                raw[t].e[p][2] = v3[2];
                raw[t].o[p][0] = v2[0];
                raw[t].o[p][1] = v2[1];
                raw[t].d0[p] = __builtin_amdgcn_raw_buffer_load_b32(rw, ok ? o : kOob, 0, 0);
                raw[t].d1[p] = __builtin_amdgcn_raw_buffer_load_b32(rw, ok ? o + 32 : kOob, 0, 0);
            }
        }
    }
}

// Position of an 8-column piece g (columns 8g .. 8g+7 of a 256-column unit) in
// the A operands: MFMA step s and lane group h.  Q8_0: step = 32-column block,
// lane group = octet of the block.  Q4_K: lane group h holds quant bytes 32h ..
// 32h+31, i.e. sub-blocks 2h (low nibbles, steps 0..3) and 2h+1 (high, 4..7),
// so piece g = 8h + s.
template <int FMT>
__device__ __forceinline__ void piece_slot(int g, int& s, int& h) {
    if constexpr (FMT == kQ4_K) {
        s = g & 7;
        h = g >> 3;
    } else {
        s = g >> 2;
        h = g & 3;
    }
}

// DPP lane moves within 16-lane rows (no LDS round trip, unlike __shfl_xor).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                              0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes

__device__ __forceinline__ void scale_of(float m, float& sc, float& inv) {
    sc = 1.f;
    inv = 1.f;
    if (m > 0.f && m <= 3.4e38f) {
        int e = 0;
        frexpf(m, &e);   // m = f * 2^e, f in [0.5, 1)
        sc = ldexpf(1.f, 15 - e);
        inv = ldexpf(1.f, e - 15);
    }
}

// The wave's activation slice (its unit's 256 columns of every batch row):
// piece q = (batch row b, 8-column group g) of lane l is q = l + 64 i, so each
// load instruction reads two rows' 1 KiB runs.  These loads are issued before
// the weight loads: the load counter drains in issue order, so the split can
// start while the weights are still in flight.
template <int MT>
__device__ __forceinline__ void ks_load_x(const KsArgs& a, int kc0, int lane, uint4 (&xr)[4 * MT][2]) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(a.batch * a.ldx * 4));
#pragma unroll
    for (int i = 0; i < 4 * MT; ++i) {
        const int q = lane + 64 * i;
        const int b = q >> 5, g = q & 31;
        const int col = kc0 + 8 * g;
        const bool ok = b < a.batch && col < a.k;
        const uint32_t off = (uint32_t)(b * a.ldx + col) * 4;
        xr[i][0] = buf_load16<false>(rx, ok ? off : kOob);
        xr[i][1] = buf_load16<false>(rx, ok ? off + 16 : kOob);
    }
}

// 16-byte slot of A-operand lane (row i, group h) for MFMA step s inside its
// 1 KiB fragment block: the row index is rotated by 2s + (h & 1).  Readers
// (one step, 64 lanes) still touch 64 distinct slots, 16 per bank group row,
// and the writers of one wave (one batch row, every step and group) spread
// over all 16 bank groups instead of all landing in one.
__device__ __forceinline__ int frag_slot(int i, int h, int s) {
    return ((i + 2 * s + (h & 1)) & 15) + 16 * h;
}

// The wave's activation slice -> fp16 (hi, lo) A fragments in the wave's LDS
// region: [step][M tile][slot][8 halves] (slot = frag_slot), then (Q4_K) the
// sub-block sums [M tile][lane][4 halves] for the 16x16x16 min product.
// rmax[i][hf] returns the largest |x| of batch row 2i + hf (uniform).
template <int FMT, int MT>
__device__ __forceinline__ void ks_prep_x(const uint4 (&xr)[4 * MT][2], uint8_t* ureg, int lane,
                                          float (&rmax)[4 * MT][2]) {
    using C = KsCfg<FMT, MT, 1>;
    const int g = lane & 31, hf = lane >> 5;
    int s, h;
    piece_slot<FMT>(g, s, h);
#pragma unroll
    for (int i = 0; i < C::PP; ++i) {
        // an empty statement that takes the piece and may touch memory: the
        // weight loads before it stay before it, and the arithmetic on the piece
        // cannot be hoisted above them
        const float4 f0 = __builtin_bit_cast(float4, xr[i][0]);
        const float4 f1 = __builtin_bit_cast(float4, xr[i][1]);
        float xv[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
        asm volatile("" : "+v"(xv[0]), "+v"(xv[1]), "+v"(xv[2]), "+v"(xv[3]), "+v"(xv[4]),
                     "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]) : : "memory");
        // largest |x| of each of the two rows (lanes 0-31: row 2i, 32-63: 2i+1)
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(xv[c]));
        m = fmaxf(m, dpp_f<kDppXor1>(m));
        m = fmaxf(m, dpp_f<kDppXor2>(m));
        m = fmaxf(m, dpp_f<kDppHalfMirror>(m));
        m = fmaxf(m, dpp_f<kDppMirror>(m));
        const int mi = __builtin_bit_cast(int, m);
        rmax[i][0] = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(mi, 0)),
                           __builtin_bit_cast(float, __builtin_amdgcn_readlane(mi, 16)));
        rmax[i][1] = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(mi, 32)),
                           __builtin_bit_cast(float, __builtin_amdgcn_readlane(mi, 48)));
        float sc, inv;
        scale_of(hf ? rmax[i][1] : rmax[i][0], sc, inv);
        const int b = 2 * i + hf;
        const int t = b >> 3, ih = 2 * (b & 7);
        f16x8 hi, lo;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float v = xv[c] * sc;
            const _Float16 vh = (_Float16)v;
            hi[c] = vh;
            lo[c] = (_Float16)(v - (float)vh);
        }
        uint8_t* frag = ureg + (s * MT + t) * 1024;
        *reinterpret_cast<f16x8*>(frag + frag_slot(ih, h, s) * 16) = hi;
        *reinterpret_cast<f16x8*>(frag + frag_slot(ih + 1, h, s) * 16) = lo;
        if constexpr (FMT == kQ4_K) {
            // sub-block jb = g / 4 is pieces 4jb .. 4jb+3: four consecutive lanes
            float sblk = ((xv[0] + xv[1]) + (xv[2] + xv[3])) + ((xv[4] + xv[5]) + (xv[6] + xv[7]));
            sblk += dpp_f<kDppXor1>(sblk);
            sblk += dpp_f<kDppXor2>(sblk);
            if ((g & 3) == 0) {
                const int jb = g >> 2, hq = jb >> 2;
                const float v = sblk * (sc * (1.f / 32.f));
                const _Float16 vh = (_Float16)v;
                _Float16* mb = reinterpret_cast<_Float16*>(ureg + C::FRAG + t * 512);
                mb[(ih + 16 * hq) * 4 + (jb & 3)] = vh;
                mb[(ih + 1 + 16 * hq) * 4 + (jb & 3)] = (_Float16)(v - (float)vh);
            }
        }
    }
    if constexpr (FMT == kQ4_K) {
        // k = 8..15 of the 16x16x16 min product (lane groups 2, 3) are zero
#pragma unroll
        for (int t = 0; t < MT; ++t)
            if (lane < 32)
                *reinterpret_cast<uint2*>(ureg + C::FRAG + t * 512 + (32 + lane) * 8) = make_uint2(0, 0);
    }
    // the wave reads these fragments itself: LDS operations of one wave complete
    // in issue order, so only the compiler must keep the reads after the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int FMT, int MT, int T>
__device__ __forceinline__ void ks_products(const uint8_t* ureg, const KsRaw<FMT> (&raw)[T],
                                            int lane, int h, f32x4 (&acc)[T][MT]) {
    using C = KsCfg<FMT, MT, T>;
    f16x8 aop[8][MT];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int t = 0; t < MT; ++t)
            aop[s][t] = *reinterpret_cast<const f16x8*>(ureg + (s * MT + t) * 1024 +
                                                        frag_slot(lane & 15, h, s) * 16);
    if constexpr (FMT == kQ4_K) {
        f16x4 amin[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t)
            amin[t] = *reinterpret_cast<const f16x4*>(ureg + C::FRAG + t * 512 + lane * 8);
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            const KsRaw<kQ4_K>& r = raw[tt];
            const float d = half_bits_to_float(r.hd.x);
            const float dmin = half_bits_to_float(r.hd.x >> 16);
            const Q4KScales scl = q4k_unpack(r.hd.y, r.hd.z, r.hd.w);
            uint32_t sc0, sc1, m_unused;
            q4k_sub(scl, 2 * h, sc0, m_unused);
            q4k_sub(scl, 2 * h + 1, sc1, m_unused);
            const uint32_t qw[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
            f32x4 dsb[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) dsb[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint32_t scj = s < 4 ? sc0 : sc1;
                const _Float16 sch = (_Float16)(float)scj;
                const _Float16 msch = (_Float16)(-1024.f * (float)scj);
                const f16x2 sc2 = {sch, sch}, msc2 = {msch, msch};
                const uint32_t w0 = qw[2 * (s & 3)], w1 = qw[2 * (s & 3) + 1];
                const uint32_t n0 = s < 4 ? w0 & 0x0F0F0F0Fu : (w0 >> 4) & 0x0F0F0F0Fu;
                const uint32_t n1 = s < 4 ? w1 & 0x0F0F0F0Fu : (w1 >> 4) & 0x0F0F0F0Fu;
                uint32_t b4[4];
                q4x4_to_f16(n0, sc2, msc2, b4[0], b4[1]);
                q4x4_to_f16(n1, sc2, msc2, b4[2], b4[3]);
                const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(b4[0], b4[1], b4[2], b4[3]));
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    dsb[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[s][t], bop, dsb[t], 0, 0, 0);
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
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const f32x4 dmn = __builtin_amdgcn_mfma_f32_16x16x16f16(amin[t], mop,
                                                                        f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                acc[tt][t] += d * dsb[t] - (32.f * dmin) * dmn;
            }
        }
    } else {
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            const KsRaw<kQ8_0>& r = raw[tt];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t b4[4];
                q8x4_to_f16(__builtin_amdgcn_alignbyte(r.e[p][1], r.e[p][0], 2), b4[0], b4[1]);
                q8x4_to_f16(__builtin_amdgcn_alignbyte(r.e[p][2], r.e[p][1], 2), b4[2], b4[3]);
                const f16x8 be = __builtin_bit_cast(f16x8, make_uint4(b4[0], b4[1], b4[2], b4[3]));
                q8x4_to_f16(r.o[p][0], b4[0], b4[1]);
                q8x4_to_f16(r.o[p][1], b4[2], b4[3]);
                const f16x8 bo = __builtin_bit_cast(f16x8, make_uint4(b4[0], b4[1], b4[2], b4[3]));
                const float d0 = half_bits_to_float(r.d0[p]);
                const float d1 = half_bits_to_float(r.d1[p] >> 16);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const f32x4 de = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[2 * p][t], be,
                                                                           f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    const f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[2 * p + 1][t], bo,
                                                                           f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    acc[tt][t] += d0 * de + d1 * dd;
                }
            }
        }
    }
}

template <int FMT, int MT, int T, bool PF>
__global__ __launch_bounds__(256) void gemv_ks_kernel(const KsArgs a) {
    using C = KsCfg<FMT, MT, T>;
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, h = lane >> 4;
    const int tile = (int)blockIdx.x / a.parts;
    const int part = (int)blockIdx.x % a.parts;
    const int64_t r0 = (int64_t)tile * C::ROWS;
    const int unit = part * kKsWaves + wave;
    const bool live = unit < a.nunit;
    uint8_t* ureg = lds + wave * C::UNIT;

    // 1. the wave's activation slice (cache-resident), then its weight bytes,
    //    all requested before any arithmetic (PF: the split of step 2 first)
    uint4 xr[4 * MT][2];
    ks_load_x<MT>(a, unit * kKsUnit, lane, xr);
    float rmax[4 * MT][2];
    if constexpr (PF) ks_prep_x<FMT, MT>(xr, ureg, lane, rmax);
    KsRaw<FMT> raw[T];
    ks_load_w<FMT, T>(a, r0, unit, live, j, h, raw);
    __builtin_amdgcn_sched_barrier(0);
    // 2. activation pairs of the wave's unit
    if constexpr (!PF) ks_prep_x<FMT, MT>(xr, ureg, lane, rmax);
    // 3. products of this wave's unit
    f32x4 acc[T][MT];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (live) ks_products<FMT, MT, T>(ureg, raw, lane, h, acc);
    // 4. D rows 4h .. 4h+3 of lane (j, h) = (batch 8m + 2h: hi, lo), (batch
    //    8m + 2h + 1: hi, lo), i.e. rows 2i, 2i + 1 of piece index i = 4m + h;
    //    each scaled back by the wave's own 2^-S_b
    float2* red = reinterpret_cast<float2*>(ureg);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float m0 = rmax[4 * m][0], m1 = rmax[4 * m][1];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            if (h == q) {
                m0 = rmax[4 * m + q][0];
                m1 = rmax[4 * m + q][1];
            }
        }
        float sc, inv0, inv1;
        scale_of(m0, sc, inv0);
        scale_of(m1, sc, inv1);
#pragma unroll
        for (int t = 0; t < T; ++t)
            red[(t * MT + m) * 64 + lane] = make_float2((acc[t][m][0] + acc[t][m][1]) * inv0,
                                                        (acc[t][m][2] + acc[t][m][3]) * inv1);
    }
    __syncthreads();

    constexpr int SLOTS = T * MT * 64;
    constexpr int SPT = (SLOTS + 255) / 256;
    float v0[SPT], v1[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int q = tid + 256 * i;
        v0[i] = v1[i] = 0.f;
        if (SLOTS % 256 == 0 || q < SLOTS) {
#pragma unroll
            for (int w = 0; w < kKsWaves; ++w) {
                const float2 v = reinterpret_cast<const float2*>(lds + w * C::UNIT)[q];
                v0[i] += v.x;
                v1[i] += v.y;
            }
        }
    }
    if (a.parts == 1) {
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int q = tid + 256 * i;
            if (SLOTS % 256 == 0 || q < SLOTS) {
                const int ln = q & 63, m = (q >> 6) % MT, t = (q >> 6) / MT;
                const int64_t row = r0 + 16 * t + (ln & 15);
                const int b0 = 8 * m + 2 * (ln >> 4);
                if (row < a.n) {
                    if (b0 < a.batch) a.y[(int64_t)b0 * a.ldy + row] = v0[i];
                    if (b0 + 1 < a.batch) a.y[(int64_t)(b0 + 1) * a.ldy + row] = v1[i];
                }
            }
        }
        return;
    }
    // K parts: publish this part's sums with device-coherent stores, wait for
    // them to complete, then count the part on the tile's counter.
    constexpr int PB = 8 * MT * C::ROWS;   // floats of one part
    float* mine = a.part + ((int64_t)tile * a.parts + part) * PB;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int q = tid + 256 * i;
        if (SLOTS % 256 == 0 || q < SLOTS) {
            const int ln = q & 63, m = (q >> 6) % MT, t = (q >> 6) / MT;
            const int rr = 16 * t + (ln & 15);
            const int b0 = 8 * m + 2 * (ln >> 4);
            __hip_atomic_store(mine + b0 * C::ROWS + rr, v0[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(mine + (b0 + 1) * C::ROWS + rr, v1[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(a.ctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)a.parts - 1;
    __syncthreads();
    if (!s_last) return;
    // last part of the tile: sum the parts in part order
    const float* tp = a.part + (int64_t)tile * a.parts * PB;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int q = tid + 256 * i;
        if (SLOTS % 256 == 0 || q < SLOTS) {
            const int ln = q & 63, m = (q >> 6) % MT, t = (q >> 6) / MT;
            const int rr = 16 * t + (ln & 15);
            const int64_t row = r0 + rr;
            const int b0 = 8 * m + 2 * (ln >> 4);
            // eight parts' loads in flight at a time (an index past the last
            // part re-reads the last one and is not added), summed in part order
            float s0 = 0.f, s1 = 0.f;
            for (int p0 = 0; p0 < a.parts; p0 += 8) {
                float v0p[8], v1p[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float* src = tp + min(p0 + u, a.parts - 1) * PB + b0 * C::ROWS + rr;
                    v0p[u] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    v1p[u] = __hip_atomic_load(src + C::ROWS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (p0 + u < a.parts) {
                        s0 += v0p[u];
                        s1 += v1p[u];
                    }
                }
            }
            if (row < a.n) {
                if (b0 < a.batch) a.y[(int64_t)b0 * a.ldy + row] = s0;
                if (b0 + 1 < a.batch) a.y[(int64_t)(b0 + 1) * a.ldy + row] = s1;
            }
        }
    }
    if (tid == 0) __hip_atomic_store(a.ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int ks_cus() {
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

template <int FMT, int MT, int T>
hipError_t ks_launch(KsArgs& a, hipStream_t s) {
    using C = KsCfg<FMT, MT, T>;
    const int64_t wgs = (int64_t)a.tiles * a.parts;
    if (FMT == kQ4_K && wgs > ks_cus())
        hipLaunchKernelGGL((gemv_ks_kernel<FMT, MT, T, true>), dim3((unsigned)wgs), dim3(256),
                           C::kLds, s, a);
    else
        hipLaunchKernelGGL((gemv_ks_kernel<FMT, MT, T, false>), dim3((unsigned)wgs), dim3(256),
                           C::kLds, s, a);
    return hipGetLastError();
}

}  // namespace

bool gemv_ks_plan(int type, int64_t n, int64_t k, int batch, size_t ws_bytes, GemvKsPlan& p) {
    if ((type != kQ4_K && type != kQ8_0) || k % kKsUnit != 0 || batch < 1 || batch > 16 || n < 1)
        return false;
    const int mt = batch > 8 ? 2 : 1;
    const int64_t nunit = k / kKsUnit;
    const int64_t parts = (nunit + kKsWaves - 1) / kKsWaves;
    const int64_t cus = ks_cus();
    // tallest row tile that still gives every compute unit a workgroup
    const int tmax = type == kQ4_K ? 4 : 2;
    int t = tmax;
    while (t > 1 && (n + 16 * t - 1) / (16 * t) * parts < cus) t /= 2;
    const int64_t tiles = (n + 16 * t - 1) / (16 * t);
    if (tiles * parts > INT32_MAX / 2) return false;
    size_t need = kCtrlBytes;
    if (parts > 1) {
        if (tiles > kKsMaxSplitTiles) return false;
        need = kCtrlBytes + (size_t)tiles * parts * 8 * mt * 16 * t * 4;
    }
    if (need > ws_bytes) return false;
    p.t = t;
    p.mt = mt;
    p.tiles = (int)tiles;
    p.parts = (int)parts;
    p.ws_bytes = need;
    // Batch 1: Q4_K matrices of more than one round of workgroups that the
    // vector-unit kernel would walk as few 8-row tiles with long K (under two
    // per compute unit, four or more 2048-wide chunks: 2560 x 9728 9.9 against
    // 10.3 us).  Elsewhere that kernel, four workgroups per compute unit, is as
    // fast or faster (9728 x 2560 8.0 against 9.1 us, 5120 x 17408 20.5
    // against 21.7, 6144 x 2048 5.1 against 7.6, 65536 x 2048 22.8 against
    // 25.6); the 1 MB Q8_0 1024 x 1024 stays there too (3.9 against 4.5 us).
    const int64_t stream_tiles = (n + 7) / 8, stream_chunks = (k + 2047) / 2048;
    p.b1 = type == kQ4_K && tiles * parts > cus && stream_tiles < 2 * cus && stream_chunks >= 4;
    return true;
}

size_t gemv_ks_ws_bytes(int type, int64_t n, int64_t k, int batch) {
    GemvKsPlan p;
    return gemv_ks_plan(type, n, k, batch, (size_t)-1, p) ? p.ws_bytes : 0;
}

hipError_t launch_gemv_ks(int type, const GemvDesc& d, int batch, const GemvKsPlan& p, void* ws,
                          hipStream_t s) {
    KsArgs a{};
    a.w = static_cast<const uint8_t*>(d.w);
    a.x = d.x;
    a.y = d.y;
    a.ctr = static_cast<uint32_t*>(ws);
    a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCtrlBytes);
    a.n = d.n;
    a.ldx = d.ldx;
    a.ldy = d.ldy;
    a.rb = (uint32_t)row_bytes(type, d.k);
    a.k = (int32_t)d.k;
    a.nunit = (int32_t)(d.k / kKsUnit);
    a.tiles = p.tiles;
    a.parts = p.parts;
    a.batch = batch;
    if (type == kQ4_K) {
        if (p.mt == 1)
            return p.t == 4 ? ks_launch<kQ4_K, 1, 4>(a, s)
                            : p.t == 2 ? ks_launch<kQ4_K, 1, 2>(a, s) : ks_launch<kQ4_K, 1, 1>(a, s);
        return p.t == 4 ? ks_launch<kQ4_K, 2, 4>(a, s)
                        : p.t == 2 ? ks_launch<kQ4_K, 2, 2>(a, s) : ks_launch<kQ4_K, 2, 1>(a, s);
    }
    if (p.mt == 1) return p.t == 2 ? ks_launch<kQ8_0, 1, 2>(a, s) : ks_launch<kQ8_0, 1, 1>(a, s);
    return p.t == 2 ? ks_launch<kQ8_0, 2, 2>(a, s) : ks_launch<kQ8_0, 2, 1>(a, s);
}

}  // namespace ggq
