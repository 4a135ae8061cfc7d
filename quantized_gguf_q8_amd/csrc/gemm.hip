// gemm.hip -- quant_gemm: prompt-batch product C[M][N] = A[M][K] * W[N][K]^T with
// W in Q8_0 / Q4_K blocks (phobos-bench pp<N>, Phobos README "Command-Line
// Tools"; the pages report prompt processing as their weaker path).
//
// This is the one dense contraction on the path, so it runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//  1. prep   : A fp32 -> bf16 (round to nearest even) into the workspace, K
//              padded with zeros to a multiple of 256 and M to a multiple of
//              16, stored in MFMA fragment order: for each 64-wide K step, each
//              group of 16 rows and each 32-wide half, the 64 lanes' 8-element
//              fragments lie in one contiguous KiB.  A fragment load is then one
//              fully used, contiguous KiB (8 cache lines) instead of 16 half
//              lines, which halves the work of the vector memory pipeline that
//              bounds this kernel.
//  2. main   : a workgroup of WV waves owns a (64*WV) x BN tile of C; wave w owns
//              rows 64w .. 64w+63 and all BN = 16*NT columns (4 x NT MFMA
//              sub-tiles, accumulators in registers).  Per 64-wide K step:
//              * the W tile (BN rows x 64) is decoded from its blocks to bf16
//                exactly once per workgroup, spread evenly over the waves, into
//                one of two LDS buffers; every wave reads all of it;
//              * each wave loads its own A fragments straight from the bf16 copy
//                (no sharing between waves, so no LDS round trip), one step
//                ahead of the MFMAs that use them;
//              * the next step's raw W bytes are fetched while this step's MFMAs
//                run, then decoded into the other buffer: one barrier per step.
//              With 8 waves (two per SIMD) one wave's decode overlaps the other
//              wave's MFMAs.  The 16-byte chunks of an LDS row are XOR-permuted
//              by row (swz below), so fragment reads and decode stores both
//              land on distinct bank groups.
//              Column tiles may overlap (stride < BN) so the tile count fits the
//              256 compute units; overlapped columns are computed twice, stored
//              once.  Rows past M and N are clamped to the last valid row: they
//              compute finite values that are never stored.
//  3. reduce : long K may be split over S workgroups writing fp32 partials; they
//              are summed in split order (deterministic, no atomics).
// Rounding: A and the decoded weights are each rounded once to bf16 (relative
// error <= 2^-9 each); products are exact in fp32 and sums accumulate in fp32.
#include "ggq_device.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kKAlign = 256;
constexpr int kBK = 64;            // K per step
constexpr int kLRow = kBK;         // bf16 per LDS row: 128 bytes

// LDS rows hold eight 16-byte chunks, chunk c of row r at slot c ^ swz(r).  A
// fragment read (16 lanes: rows r0..r0+15, one chunk) then covers the 16 slots
// of a 256-byte bank window once (rows of one parity get distinct swz), and a
// Q4_K decode store (16 lanes: four rows, four chunks each) too (rows 4m and
// 4m+2 differ in bit 2 of swz, so their chunks 0-3 / 4-7 land on disjoint
// slots).
__host__ __device__ constexpr int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
constexpr int kDW = 4;             // steps of raw W bytes in flight

inline int64_t kpad(int64_t k) { return (k + kKAlign - 1) / kKAlign * kKAlign; }

// Hardware round-to-nearest-even conversion of two floats to packed bf16.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__host__ __device__ inline int64_t mpad(int64_t m) { return (m + 15) / 16 * 16; }

// Byte offset of the fragment (16-row group g, K step st, half h, lane l) in the
// fragment-ordered copy with `groups` row groups.
__host__ __device__ inline int64_t frag_offset(int64_t st, int64_t g, int h, int l, int64_t groups) {
    return (((st * groups + g) * 2 + h) * 64 + l) * 16;
}

// One thread per 16-byte fragment piece, in output order: a wave writes 1 KiB
// contiguously and reads 16 rows x 128 contiguous bytes.
__global__ __launch_bounds__(256) void prep_bf16_kernel(const float* __restrict__ a, int64_t lda,
                                                        int64_t m, int64_t k, int64_t kp,
                                                        uint16_t* __restrict__ out) {
    const int64_t groups = mpad(m) / 16;
    const int64_t pieces = groups * 16 * kp / 8;
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= pieces) return;
    const int l = (int)(p % 64);
    const int h = (int)((p / 64) % 2);
    const int64_t g = (p / 128) % groups;
    const int64_t st = p / 128 / groups;
    const int64_t row = g * 16 + l % 16;
    const int64_t col = st * kBK + 32 * h + 8 * (l / 16);
    float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
    if (row < m && col < k) {   // k is a multiple of 32
        const float4* src = reinterpret_cast<const float4*>(a + row * lda + col);
        v0 = src[0];
        v1 = src[1];
    }
    uint4 o;
    o.x = cvt_bf16x2(v0.x, v0.y);
    o.y = cvt_bf16x2(v0.z, v0.w);
    o.z = cvt_bf16x2(v1.x, v1.y);
    o.w = cvt_bf16x2(v1.z, v1.w);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(out) + frag_offset(st, g, h, l, groups)) = o;
}

// One decode unit = 16 weights of one W row in the current step.
//  Q4_K: the step is 64-weight group g = (k0/64)%4 of super-block k0/256; unit u
//        (0..3) holds quant bytes 32g + 8u .. +7, i.e. step columns 8u + i (low
//        nibbles, sub-block 2g) and 32 + 8u + i (high nibbles, sub-block 2g+1).
//  Q8_0: unit h (0..3) is half h%2 of block k0/32 + h/2: step columns 16h .. +15.
template <int FMT>
struct RawUnit;
template <>
struct RawUnit<kQ4_K> {
    u32x4 hdr;   // d | dmin, packed scales
    uint32_t q0, q1;
};
template <>
struct RawUnit<kQ8_0> {
    uint32_t d;      // scale bits (low half)
    u32x4 x;         // 16 bytes from the dword-aligned start of the quants
    uint32_t x4;     // the two bytes after them
    uint32_t sh;     // byte misalignment of the quants (0 or 2)
};

struct WView {
    __amdgpu_buffer_rsrc_t rsrc;   // over the whole matrix
    int64_t n, rb, nblk;           // rows, bytes per row, Q8_0 blocks per row
};

template <int FMT>
__device__ __forceinline__ void load_unit(const WView& v, int64_t row, int k0, int u,
                                          RawUnit<FMT>& r) {
    row = row < v.n ? row : v.n - 1;
    const uint32_t rowoff = (uint32_t)(row * v.rb);
    if constexpr (FMT == kQ4_K) {
        const uint32_t sb = rowoff + (uint32_t)(k0 / 256) * kQ4Bytes;
        r.hdr = __builtin_amdgcn_raw_buffer_load_b128(v.rsrc, sb, 0, 0);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(
            v.rsrc, sb + 16 + 32 * ((k0 / 64) & 3) + 8 * u, 0, 0);
        r.q0 = q.x;
        r.q1 = q.y;
    } else {
        int64_t blk = k0 / 32 + (u >> 1);
        blk = blk < v.nblk ? blk : v.nblk - 1;   // K tail: finite weights times zero A
        const uint32_t b = rowoff + (uint32_t)blk * kQ8Bytes;
        const uint32_t o = b + 2 + 16 * (u & 1);
        const uint32_t base = o & ~3u;
        r.sh = o & 3u;
        r.d = __builtin_amdgcn_raw_buffer_load_b16(v.rsrc, b, 0, 0);
        r.x = __builtin_amdgcn_raw_buffer_load_b128(v.rsrc, base, 0, 0);
        // only the first two bytes of the next dword are used (when sh == 2); a
        // 2-byte load keeps the read inside the block
        r.x4 = __builtin_amdgcn_raw_buffer_load_b16(v.rsrc, base + 16, 0, 0);
    }
}

// Four quant bytes v -> w = a*(1024 + v) + c as four bf16 (two packed words).
// A byte permute places each byte under the exponent byte 0x64, which makes the
// exact fp16 value 1024 + v (two per instruction); one mixed-precision FMA per
// weight then gives a*v + b with c = b - 1024a.
__device__ __forceinline__ void decode4(uint32_t v, float a, float c, uint32_t& o0, uint32_t& o1) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    constexpr uint32_t e = 0x64646464u;
    const h2 p0 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(e, v, 0x04010400u));
    const h2 p1 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(e, v, 0x04030402u));
    o0 = cvt_bf16x2(__builtin_fmaf(a, (float)p0.x, c), __builtin_fmaf(a, (float)p0.y, c));
    o1 = cvt_bf16x2(__builtin_fmaf(a, (float)p1.x, c), __builtin_fmaf(a, (float)p1.y, c));
}

// Decode one unit into 16 bf16 weights of LDS row `dst` (bf16 elements, chunks
// permuted by f = swz(row)).  For
// Q4_K, g = (step) % 4 is the step's 64-weight group of its super-block; the
// callers pass it as a constant so that the scale and min extraction of the two
// sub-blocks 2g, 2g+1 is a handful of fixed bit-field reads.
template <int FMT>
__device__ __forceinline__ void store_unit(const RawUnit<FMT>& r, int u, int g, uint16_t* dst,
                                           int f) {
    if constexpr (FMT == kQ4_K) {
        // packed scales s[0..11] = hdr.y, hdr.z, hdr.w.  Sub-block j < 4: scale
        // s[j] & 63, min s[j+4] & 63; j >= 4: scale low nibble of s[j+4] with the
        // top two bits of s[j-4], min high nibble of s[j+4] with those of s[j].
        uint32_t sc0, m0, sc1, m1;
        if (g < 2) {
            // hdr.w is not needed here, but its register must stay this load's
            // until the load is waited for: handed to the allocator as free, it
            // is reused at once and the write waits for every load in flight
            asm volatile("" : : "v"(r.hdr.w));
            const int sh = 16 * g;
            sc0 = (r.hdr.y >> sh) & 63u;
            sc1 = (r.hdr.y >> (sh + 8)) & 63u;
            m0 = (r.hdr.z >> sh) & 63u;
            m1 = (r.hdr.z >> (sh + 8)) & 63u;
        } else {
            const int sh = 16 * (g - 2);
            sc0 = ((r.hdr.w >> sh) & 15u) | (((r.hdr.y >> (sh + 6)) & 3u) << 4);
            sc1 = ((r.hdr.w >> (sh + 8)) & 15u) | (((r.hdr.y >> (sh + 14)) & 3u) << 4);
            m0 = ((r.hdr.w >> (sh + 4)) & 15u) | (((r.hdr.z >> (sh + 6)) & 3u) << 4);
            m1 = ((r.hdr.w >> (sh + 12)) & 15u) | (((r.hdr.z >> (sh + 14)) & 3u) << 4);
        }
        const float d = half_bits_to_float(r.hdr.x);
        const float dmin = half_bits_to_float(r.hdr.x >> 16);
        const float a0 = d * (float)sc0, a1 = d * (float)sc1;
        const float c0 = -dmin * (float)m0 - 1024.f * a0;
        const float c1 = -dmin * (float)m1 - 1024.f * a1;
        const uint32_t qw[2] = {r.q0, r.q1};
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            decode4(opaque(qw[i] & 0x0F0F0F0Fu), a0, c0, lo[2 * i], lo[2 * i + 1]);
            decode4(opaque((qw[i] >> 4) & 0x0F0F0F0Fu), a1, c1, hi[2 * i], hi[2 * i + 1]);
        }
        *reinterpret_cast<uint4*>(dst + 8 * (u ^ f)) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<uint4*>(dst + 8 * ((4 + u) ^ f)) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    } else {
        (void)g;
        // (q ^ 0x80) read as an unsigned byte is u = q + 128, and d*q =
        // d*(1024 + u) - 1152d exactly (both products fit in fp32's mantissa).
        const float d = half_bits_to_float(r.d);
        const float c = -1152.f * d;
        const uint32_t xs[5] = {r.x.x, r.x.y, r.x.z, r.x.w, r.x4};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            decode4(__builtin_amdgcn_alignbyte(xs[i + 1], xs[i], r.sh) ^ 0x80808080u, d, c,
                    o[2 * i], o[2 * i + 1]);
        *reinterpret_cast<uint4*>(dst + 8 * ((2 * u) ^ f)) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(dst + 8 * ((2 * u + 1) ^ f)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

template <int WV, int NT>
struct GemmShape {
    static constexpr int THREADS = 64 * WV;
    static constexpr int BM = 64 * WV;
    static constexpr int BN = 16 * NT;
    static constexpr int UNITS = BN * (kBK / 16);            // decode units per step
    static constexpr int UPW = (UNITS + WV - 1) / WV;       // per wave
    static constexpr int UPT = (UPW + 63) / 64;             // per thread
    // bf16 elements per buffer: BN rows plus one row that absorbs the stores of
    // lanes without a decode unit (so the decode has no branch)
    static constexpr int kBuf = (BN + 1) * kLRow;
    static constexpr int kLds = 2 * kBuf * 2;               // bytes
};

struct GemmArgs {
    const uint8_t* w;
    const uint16_t* abf;   // fragment-ordered bf16 copy of A (see frag_offset)
    float* c;              // output (S == 1) or partials [S][M][N]
    int64_t n, k, rb, kp, m, ldc;
    int32_t stride;        // column-tile stride (<= BN)
    int32_t tiles_m, tiles_n, splits;
    int32_t ksteps_per_split;
};

template <int FMT, int WV, int NT>
__global__ __launch_bounds__(64 * WV) void gemm_kernel(const GemmArgs p) {
    using S = GemmShape<WV, NT>;
    extern __shared__ __align__(16) uint16_t wl[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // tile index: split-K fastest, then M, then N
    int t = blockIdx.x;
    const int split = t % p.splits;
    t /= p.splits;
    const int tm = t % p.tiles_m;
    const int tn = t / p.tiles_m;
    const int64_t m0 = (int64_t)tm * S::BM + 64 * wave;
    const int64_t n0 = (int64_t)tn * p.stride;
    const int kstep0 = split * p.ksteps_per_split;
    const int nk = min(p.ksteps_per_split, (int)(p.kp / kBK) - kstep0);

    WView wv;
    wv.rsrc = make_rsrc(p.w, (uint32_t)(p.n * p.rb));
    wv.n = p.n;
    wv.rb = p.rb;
    wv.nblk = p.k / 32;

    f32x4 acc[4][NT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A fragments: sub-tile i, lane l -> row m0 + 16i + l%16, columns 8(l/16) .. +7
    // of each 32-wide half of the step.  Row groups past the padded M read the
    // last group (finite values, never stored).
    const int64_t groups = mpad(p.m) / 16;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.abf, (uint32_t)(groups * 16 * p.kp * 2));
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t g = (m0 + 16 * i) / 16;
        g = g < groups ? g : groups - 1;
        aoff[i] = (uint32_t)frag_offset(0, g, 0, lane, groups);
    }
    const uint32_t astep = (uint32_t)(groups * 2048);   // bytes per K step
    bf16x8 af[2][4], an[2][4];
    // decode units of this thread: wave w takes units UPW*w .. UPW*w + UPW-1,
    // unit q = row q / 4, part q % 4: four consecutive lanes read one row's bytes
    // of the step together, so a load instruction touches few cache lines
    RawUnit<FMT> ru[kDW][S::UPT];

    // The loop body is unrolled kDW = 4 times so that every register ring index
    // and every step's position in its super-block is a compile-time constant;
    // the host makes a split's step count a multiple of 4, so no step needs a
    // branch or a variable wait count.  Loads ahead of the last step read the
    // last step again and are never used.
    static_assert(kDW == 4, "the decode takes a step's super-block group from the unroll index");
    const int nsteps = nk;
    // The step offset is uniform and goes in the scalar offset, so an A load
    // costs no vector instruction.  The load after the last step (issued by the
    // last step, never used) reads the last step again.
    auto load_a = [&](int ks, bf16x8 (&dst)[2][4]) {
        const uint32_t kb = (uint32_t)(kstep0 + min(ks, nk - 1)) * astep;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[h][i] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[i] + 1024 * h, kb, 0));
    };
    // Lanes past a wave's share load a valid unit too (and never store it).
    auto unit_of = [&](int i) {
        const int q = S::UPW * wave + min(lane + 64 * i, S::UPW - 1);
        return min(q, S::UNITS - 1);
    };
    auto load_w = [&](int ks, RawUnit<FMT> (&dst)[S::UPT]) {
        const int step = kstep0 + min(ks, nk - 1);
#pragma unroll
        for (int i = 0; i < S::UPT; ++i) {
            const int q = unit_of(i);
            load_unit<FMT>(wv, n0 + q / 4, step * kBK, q % 4, dst[i]);
        }
    };
    // g = the step's index mod 4, a constant at every call (kstep0 and the
    // unrolled loop's base step are multiples of 4, and nk is too, so no step
    // is clamped)
    auto store_w = [&](int g, const RawUnit<FMT> (&src)[S::UPT], uint16_t* buf) {
#pragma unroll
        for (int i = 0; i < S::UPT; ++i) {
            const int qi = lane + 64 * i;
            const int q = S::UPW * wave + qi;
            const int row = (qi < S::UPW && q < S::UNITS) ? q / 4 : S::BN;
            store_unit<FMT>(src[i], q % 4, g, buf + row * kLRow, swz(row));
        }
    };

    if (nk > 0) {
        // A first, as in the loop: at the loop head the A fragments are then
        // followed by weight loads on every path into it, and the first
        // step's wait for them need not drain the weight prefetch
        load_a(0, af);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < kDW; ++d) load_w(d, ru[d]);
        store_w(0, ru[0], wl);
    }
    __syncthreads();
    for (int ks0 = 0; ks0 < nsteps; ks0 += kDW) {
#pragma unroll
        for (int d = 0; d < kDW; ++d) {
            const int ks = ks0 + d;
            bf16x8 (&acur)[2][4] = (d & 1) ? an : af;
            bf16x8 (&anext)[2][4] = (d & 1) ? af : an;
            // fetch the next step's A fragments, then refill ring slot d (it held
            // step ks, decoded during the previous step) with step ks + kDW.  The
            // order matters: loads complete in issue order as far as the wait
            // counter is concerned, so A issued before the weights lets the next
            // step's MFMAs wait only for weights fetched steps earlier.
            load_a(ks + 1, anext);
            load_w(ks + kDW, ru[d]);
            // row 16j + (lane & 15), chunk (lane >> 4) + 4h; swz depends on the
            // row's low four bits only, and chunk ^ swz = ((lane >> 4) ^ swz) ^ 4h
            const uint16_t* bbase = wl + (d & 1) * S::kBuf + (lane & 15) * kLRow;
            const int c0 = (lane >> 4) ^ swz(lane & 15);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(
                        bbase + 16 * j * kLRow + 8 * (c0 ^ (4 * h)));
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur[h][i], bfr,
                                                                            acc[i][j], 0, 0, 0);
                }
            }
            store_w((d + 1) % kDW, ru[(d + 1) % kDW], wl + ((d + 1) & 1) * S::kBuf);
            __syncthreads();
        }
    }

    // D[i][j]: lane holds rows 4*(lane/16) + r, column lane%16 of each sub-tile.
    const int64_t nend = min(n0 + p.stride, p.n);
    float* out = p.splits == 1 ? p.c : p.c + (int64_t)split * p.m * p.n;
    const int64_t ld = p.splits == 1 ? p.ldc : p.n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t col = n0 + 16 * j + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 16 * i + 4 * (lane >> 4) + r;
                if (row < p.m && col < nend) out[row * ld + col] = acc[i][j][r];
            }
        }
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int64_t m, int64_t n,
                                                            float* __restrict__ c, int64_t ldc) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= m * n) return;
    const int64_t row = i / n, col = i % n;
    float s = 0.f;
    for (int q = 0; q < splits; ++q) s += part[q * m * n + i];
    c[row * ldc + col] = s;
}

// The same sums for four consecutive outputs of a row per thread (n and ldc
// multiples of 4, part and c 16-byte aligned), the parts added from zero in
// split order as above; up to eight parts are loaded before the first add.
__global__ __launch_bounds__(256) void splitk_reduce4_kernel(const float4* __restrict__ part,
                                                             int splits, int64_t m, int64_t n,
                                                             float* __restrict__ c, int64_t ldc) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t mn4 = m * n / 4;
    if (i >= mn4) return;
    const int64_t row = 4 * i / n, col = 4 * i % n;
    float4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        if (q < splits) v[q] = part[q * mn4 + i];
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (q < splits) {
            s.x += v[q].x;
            s.y += v[q].y;
            s.z += v[q].z;
            s.w += v[q].w;
        }
    }
    for (int q = 8; q < splits; ++q) {
        const float4 t = part[q * mn4 + i];
        s.x += t.x;
        s.y += t.y;
        s.z += t.z;
        s.w += t.w;
    }
    *reinterpret_cast<float4*>(c + row * ldc + col) = s;
}

// Tile plan: waves per workgroup WV (rows 64*WV), column-tile width BN = 16*NT
// and stride, K splits.  The estimate is the MFMA time of the busiest compute
// unit (workgroups run in rounds over 256 units, each holding two waves per
// SIMD) plus the fp32 partial-sum traffic of a split.
struct Plan {
    int wv, nt, stride, splits, tiles_m, tiles_n;
};

constexpr int kCUs = 256;

Plan plan_for(int64_t m, int64_t n, int64_t k) {
    const int64_t ksteps = kpad(k) / kBK;
    Plan best{4, 4, 64, 1, 1, 1};
    double best_t = 1e300;
    int64_t best_wgs = 0;
    const double abytes = (double)mpad(m) * (double)kpad(k) * 2.0;
    const double afill_w = abytes > 4.0 * (1 << 20) ? 0.5 : 0.1;
    const int wvs[] = {8, 4};
    const int nts[] = {6, 5, 4, 3, 2, 1};
    for (int wv : wvs) {
        const int64_t tiles_m = (m + 64 * wv - 1) / (64 * wv);
        const int64_t slots = (int64_t)kCUs * (8 / wv);   // resident workgroups
        for (int nt : nts) {
            const int bn = 16 * nt;
            for (int stride = bn; stride >= bn / 2 && stride > 0; stride -= 4) {
                const int64_t tn = (n + stride - 1) / stride;
                for (int s = 1; s <= 8; s *= 2) {
                    if (s > 1 && ksteps / s < 8) break;
                    const int64_t kper = (ksteps + s - 1) / s;
                    const int64_t wgs = tiles_m * tn * s;
                    const int64_t rounds = (wgs + slots - 1) / slots;
                    // cycles per compute unit and round: 2048 MACs per cycle at ~50%
                    // of peak, plus the cycles to bring the tile's real A rows in
                    // at 64 bytes per cycle (each column tile re-reads its whole A
                    // block, which narrow tiles pay for many times), counted at
                    // 1/10 while the bf16 A fits one XCD's 4 MB L2 and at 1/2 when
                    // it has to come from further out; 2500 bytes per cycle of
                    // memory for split-K partials (written and read back)
                    const double mfma = (8 / wv) * (64.0 * wv) * bn * (kper * kBK) / 1024.0;
                    const double arows = (double)(mpad(m) < 64 * wv ? mpad(m) : 64 * wv);
                    const double afill = (8 / wv) * arows * (kper * kBK) * 2.0 / 64.0;
                    double t = (double)rounds * (mfma + afill_w * afill);
                    if (s > 1) t += (double)s * m * n * 8.0 / 2500.0;
                    if (t < best_t * 0.999 || (t <= best_t * 1.001 && wgs < best_wgs)) {
                        best_t = t;
                        best_wgs = wgs;
                        best = Plan{wv, nt, stride, s, (int)tiles_m, (int)tn};
                    }
                }
            }
        }
    }
    return best;
}

template <int FMT, int WV, int NT>
hipError_t launch_main(const GemmArgs& a, hipStream_t s) {
    using S = GemmShape<WV, NT>;
    const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n * a.splits);
    hipLaunchKernelGGL((gemm_kernel<FMT, WV, NT>), dim3(grid), dim3(S::THREADS), S::kLds, s, a);
    return hipGetLastError();
}

template <int FMT, int WV>
hipError_t launch_nt(const GemmArgs& a, int nt, hipStream_t s) {
    switch (nt) {
        case 6: return launch_main<FMT, WV, 6>(a, s);
        case 5: return launch_main<FMT, WV, 5>(a, s);
        case 4: return launch_main<FMT, WV, 4>(a, s);
        case 3: return launch_main<FMT, WV, 3>(a, s);
        case 2: return launch_main<FMT, WV, 2>(a, s);
        default: return launch_main<FMT, WV, 1>(a, s);
    }
}

template <int FMT>
hipError_t launch_fmt(const GemmArgs& a, const Plan& pl, hipStream_t s) {
    return pl.wv == 8 ? launch_nt<FMT, 8>(a, pl.nt, s) : launch_nt<FMT, 4>(a, pl.nt, s);
}

}  // namespace

size_t gemm_workspace_bytes(int type, int64_t m, int64_t n, int64_t k) {
    (void)type;
    const Plan pl = plan_for(m, n, k);
    size_t bytes = ((size_t)mpad(m) * (size_t)kpad(k) * 2 + 255) / 256 * 256;
    if (pl.splits > 1) bytes += (size_t)pl.splits * (size_t)m * (size_t)n * 4;
    return bytes + 256;
}

hipError_t launch_gemm(int type, const uint8_t* w, int64_t n, int64_t k, const float* a,
                       int64_t lda, int64_t m, float* c, int64_t ldc, void* ws, hipStream_t s) {
    if (gemm_mid_applies(type, m, n, k))   // its workspace (M*K bf16) fits in this one
        return launch_gemm_mid(type, w, n, k, a, lda, m, c, ldc, ws, s);
    const int64_t kp = kpad(k);
    uint16_t* abf = static_cast<uint16_t*>(ws);
    const int64_t total = mpad(m) * (kp / 8);
    hipLaunchKernelGGL(prep_bf16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a,
                       lda, m, k, kp, abf);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const Plan pl = plan_for(m, n, k);
    GemmArgs g;
    g.w = w;
    g.abf = abf;
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                           ((size_t)mpad(m) * (size_t)kp * 2 + 255) / 256 * 256);
    g.c = pl.splits == 1 ? c : part;
    g.n = n;
    g.k = k;
    g.rb = row_bytes(type, k);
    g.kp = kp;
    g.m = m;
    g.ldc = ldc;
    g.stride = pl.stride;
    g.tiles_m = pl.tiles_m;
    g.tiles_n = pl.tiles_n;
    g.splits = pl.splits;
    const int ksteps = (int)(kp / kBK);
    // a multiple of 4 steps per split (the kernel's decode takes the step's
    // position in its super-block from the unrolled loop index); ksteps is one
    g.ksteps_per_split = ((ksteps + pl.splits - 1) / pl.splits + 3) / 4 * 4;
    err = type == kQ4_K ? launch_fmt<kQ4_K>(g, pl, s) : launch_fmt<kQ8_0>(g, pl, s);
    if (err != hipSuccess || pl.splits == 1) return err;
    if (n % 4 == 0 && ldc % 4 == 0 && reinterpret_cast<uintptr_t>(c) % 16 == 0 &&
        reinterpret_cast<uintptr_t>(part) % 16 == 0)
        hipLaunchKernelGGL(splitk_reduce4_kernel, dim3((unsigned)((m * n / 4 + 255) / 256)),
                           dim3(256), 0, s, reinterpret_cast<const float4*>(part), pl.splits, m, n,
                           c, ldc);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((m * n + 255) / 256)), dim3(256),
                           0, s, part, pl.splits, m, n, c, ldc);
    return hipGetLastError();
}

}  // namespace ggq
