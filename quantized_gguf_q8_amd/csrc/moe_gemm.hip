// moe_gemm.hip -- moe_expert_gemm: the routed expert feed-forward of a
// mixture-of-experts layer at prompt batch (Phobos README opening paragraph for
// the layer; phobos-bench pp<N>, README "Command-Line Tools", for prompt
// processing through it).
//
// At a few hundred tokens every expert receives tens of (token, slot) pairs, so
// each expert's three matrices are worth reading once for all of them on the
// matrix cores (v_mfma_f32_16x16x32_bf16) rather than once per small token group.
// Five launches on the caller's stream:
//   1. group   : one workgroup counts the pairs per expert, gives each expert a
//                run of "slots" padded to a multiple of 16, writes which pair sits
//                in each slot (-1 for padding) and cuts every expert's run into
//                tiles of at most 64 slots.  Slots within an expert are handed
//                out by LDS atomics: the order can vary between calls, the
//                results cannot (a row of a matrix-core product depends only on
//                its own operands).
//   2. x->bf16 : the activation rows rounded once to bf16 (nearest even).
//   3. gate/up : per (tile, 64 rows of F): h = silu(Wg x) * (Wu x) for every slot
//                of the tile, written as bf16 in slot order.
//   4. down    : per (tile, 128 rows of H): d = Wd h, written in fp32 to the row
//                of the slot's pair.
//   5. combine : y[t] = sum_s probs[t][s] * d_(t,s) in slot order.
// Kernels 3 and 4 are the same code.  A workgroup of kMgWaves waves holds one tile;
// the tile's bf16 activations are staged through LDS 256 columns at a time and
// shared by the waves, while each wave decodes its own 16-row column tiles of
// the quantized weights straight into matrix-core operands (no LDS round trip
// for weights, no weight byte read twice).  Rounding: activations, h and the
// decoded weights are each rounded once to bf16; products accumulate in fp32.
// The result is within the prompt-GEMM tolerance of each product (8e-3 of the
// sum of |a w|), propagated through silu(g)*u.
//
// K order inside the 16x16x32 products.  Any assignment of a chunk's 256
// columns to (lane group q = lane / 16, product s, slot i) gives the same sums
// as long as both operands use it; the one here lets each lane decode weights
// from bytes it loaded itself, with the four lanes of a weight row reading
// neighbouring bytes (mg_kcol):
//   Q8_0: lanes of group q own blocks 2q and 2q+1 (columns 64q .. 64q+63);
//         product s takes columns 64q + 8s .. +7.
//   Q4_K: lanes of group q own quant bytes 16q .. 16q+15 and 64+16q .. +15 of
//         the super-block, i.e. 16 low- and 16 high-nibble weights in each of
//         the 64-weight groups q/2 and 2 + q/2; product s takes, in group
//         q/2 + 2(s/4), the nibbles (low for s%4 < 2, high after) of bytes
//         16(q%2) + 8(s%2) .. +7.
#include <type_traits>

#include "ggq_device.h"
#include "ggq_launch.h"

namespace ggq {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kPad = 16;     // slot rows per expert are padded to this
constexpr int kBM = 64;      // slots per tile (four 16-row groups)
constexpr int kKC = 256;     // columns per chunk
constexpr int kAFrag = 1024; // bytes of one 16x32 bf16 operand fragment
constexpr int kABuf = 8 * 4 * kAFrag;   // one chunk: 8 products x 4 groups
constexpr int kMgWaves = 4;  // waves per workgroup of the grouped products

__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// ---------------------------------------------------------------- layout ----
// Workspace (see mg_carve): bookkeeping ints, then x in bf16 [T][H], h in bf16
// [slots][F], and the per-pair down outputs [P][H] fp32.
struct MgWs {
    int32_t* hdr;     // [0] tiles, [1] padded slots
    int32_t* tiles;   // [tile][2]: first slot, expert << 3 | 16-row groups
    int32_t* spair;   // [slot] pair id t*top_k + s, or -1 for padding
    uint16_t* xb;     // [T][H]
    uint16_t* hb;     // [slot][F]
    float* dbuf;      // [P][H]
};

inline size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

// Slots and tiles are bounded on the host: each active expert (at most
// min(E, P)) pads fewer than 16 slots and starts at most one partial tile.
int64_t moe_gemm_slot_bound(int64_t e, int64_t p) { return p + (kPad - 1) * (e < p ? e : p); }

int64_t moe_gemm_tile_bound(int64_t e, int64_t p) {
    return (moe_gemm_slot_bound(e, p) + kBM - 1) / kBM + (e < p ? e : p);
}

size_t moe_gemm_ws_bytes(int64_t e, int64_t t, int top_k, int64_t h, int64_t f) {
    const int64_t p = t * top_k;
    const int64_t sb = moe_gemm_slot_bound(e, p), tb = moe_gemm_tile_bound(e, p);
    return al256(64) + al256((size_t)tb * 8) + al256((size_t)sb * 4) + al256((size_t)t * h * 2) +
           al256((size_t)sb * f * 2) + al256((size_t)p * h * 4);
}

namespace {

MgWs mg_carve(void* ws, int64_t e, int64_t t, int top_k, int64_t h, int64_t f) {
    const int64_t p = t * top_k;
    const int64_t sb = moe_gemm_slot_bound(e, p), tb = moe_gemm_tile_bound(e, p);
    uint8_t* b = static_cast<uint8_t*>(ws);
    MgWs m;
    m.hdr = reinterpret_cast<int32_t*>(b);
    b += al256(64);
    m.tiles = reinterpret_cast<int32_t*>(b);
    b += al256((size_t)tb * 8);
    m.spair = reinterpret_cast<int32_t*>(b);
    b += al256((size_t)sb * 4);
    m.xb = reinterpret_cast<uint16_t*>(b);
    b += al256((size_t)t * h * 2);
    m.hb = reinterpret_cast<uint16_t*>(b);
    b += al256((size_t)sb * f * 2);
    m.dbuf = reinterpret_cast<float*>(b);
    return m;
}

// ----------------------------------------------------------------- group ----
// One workgroup of 1024 threads (thread e owns expert e in the scans; E <= 1024).
__global__ __launch_bounds__(1024) void mg_group_kernel(const int32_t* __restrict__ idx, int p,
                                                        int e, MgWs ws) {
    __shared__ int32_t cnt[1024], cur[1024], first[1024];
    __shared__ int32_t wsum[16][2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    cnt[tid] = 0;
    cur[tid] = 0;
    __syncthreads();
    for (int i = tid; i < p; i += 1024) {
        int ex = idx[i];
        ex = (ex >= 0 && ex < e) ? ex : 0;
        atomicAdd(&cnt[ex], 1);
    }
    __syncthreads();
    // exclusive scans of padded slots and tiles over experts
    const int c = tid < e ? cnt[tid] : 0;
    const int rows = (c + kPad - 1) / kPad * kPad;
    const int nt = (rows + kBM - 1) / kBM;
    int a = rows, b = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int a2 = __shfl_up(a, o, 64), b2 = __shfl_up(b, o, 64);
        if (lane >= o) {
            a += a2;
            b += b2;
        }
    }
    if (lane == 63) {
        wsum[wave][0] = a;
        wsum[wave][1] = b;
    }
    __syncthreads();
    int pa = 0, pb = 0;
    for (int w = 0; w < wave; ++w) {
        pa += wsum[w][0];
        pb += wsum[w][1];
    }
    const int s0 = pa + a - rows, t0 = pb + b - nt;
    first[tid] = s0;
    if (tid < e) {
        for (int j = 0; j < nt; ++j) {
            const int r = rows - kBM * j < kBM ? rows - kBM * j : kBM;
            ws.tiles[2 * (t0 + j)] = s0 + kBM * j;
            ws.tiles[2 * (t0 + j) + 1] = (tid << 3) | (r / 16);
        }
        for (int s = c; s < rows; ++s) ws.spair[s0 + s] = -1;
    }
    if (tid == 1023) {
        ws.hdr[0] = pb + b;
        ws.hdr[1] = pa + a;
    }
    __syncthreads();
    for (int i = tid; i < p; i += 1024) {
        int ex = idx[i];
        ex = (ex >= 0 && ex < e) ? ex : 0;
        ws.spair[first[ex] + atomicAdd(&cur[ex], 1)] = i;
    }
}

// x fp32 -> bf16, 8 values per thread (count8 = T*H/8).
__global__ __launch_bounds__(256) void mg_xbf_kernel(const float* __restrict__ x, int64_t count8,
                                                     uint16_t* __restrict__ xb) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count8) return;
    const float4* src = reinterpret_cast<const float4*>(x) + 2 * i;
    const float4 v0 = src[0], v1 = src[1];
    uint4 o;
    o.x = cvt_bf16x2(v0.x, v0.y);
    o.y = cvt_bf16x2(v0.z, v0.w);
    o.z = cvt_bf16x2(v1.x, v1.y);
    o.w = cvt_bf16x2(v1.z, v1.w);
    reinterpret_cast<uint4*>(xb)[i] = o;
}

// --------------------------------------------------------- grouped GEMM ----
struct MgArgs {
    const uint8_t* w[2];     // expert-stacked matrices [E][n][rb] (NMAT of them)
    int64_t n, rb;           // rows per expert matrix, bytes per row
    int32_t k;               // columns, a multiple of 256
    int32_t ntn;             // column tiles of the grid
    const uint16_t* a;       // bf16 activation rows, k wide
    uint32_t abytes;         // size of a
    int32_t adiv;            // > 0: row of slot = pair / adiv (gate/up); 0: row = slot
    const int32_t* hdr;
    const int32_t* tiles;
    const int32_t* spair;
    uint16_t* hout;          // gate/up: bf16 h [slot][ldo]
    float* dout;             // down: fp32 [pair][ldo]
    int64_t ldo;
    // > 0: a dense product of that many activation rows (one "expert", slot i =
    // row i, tiles of 64 rows in blockIdx order); hdr, tiles and spair unused
    int32_t dense_m;
    int32_t ksplit;          // dense only: K halves (1 or 2); otherwise 1
};

// Raw bytes one lane loads per 256-column chunk of one 16-row column tile:
// Q4_K the super-block header and the 32 quant bytes of its group q; Q8_0 the
// 68 bytes of blocks 2q and 2q+1.
template <int FMT>
struct MgRaw;
template <>
struct MgRaw<kQ4_K> {
    u32x4 hdr, q0, q1;
};
template <>
struct MgRaw<kQ8_0> {
    u32x4 v0, v1, v2, v3;
    uint32_t v4;
};

template <int FMT>
__device__ __forceinline__ void mg_load(__amdgpu_buffer_rsrc_t r, uint32_t rowoff, int c, int q,
                                        MgRaw<FMT>& o) {
    if constexpr (FMT == kQ4_K) {
        const uint32_t b = rowoff == kOob ? kOob : rowoff + (uint32_t)c * kQ4Bytes;
        const uint32_t bq = rowoff == kOob ? kOob : b + 16 + 16 * q;
        o.hdr = __builtin_amdgcn_raw_buffer_load_b128(r, b, 0, 0);
        o.q0 = __builtin_amdgcn_raw_buffer_load_b128(r, bq, 0, 0);
        o.q1 = __builtin_amdgcn_raw_buffer_load_b128(r, rowoff == kOob ? kOob : bq + 64, 0, 0);
    } else {
        // dword aligned: rows and chunks start on 16 bytes, 68q on 4
        const uint32_t b = rowoff == kOob ? kOob : rowoff + (uint32_t)c * (8 * kQ8Bytes) + 68 * q;
        o.v0 = __builtin_amdgcn_raw_buffer_load_b128(r, b, 0, 0);
        o.v1 = __builtin_amdgcn_raw_buffer_load_b128(r, rowoff == kOob ? kOob : b + 16, 0, 0);
        o.v2 = __builtin_amdgcn_raw_buffer_load_b128(r, rowoff == kOob ? kOob : b + 32, 0, 0);
        o.v3 = __builtin_amdgcn_raw_buffer_load_b128(r, rowoff == kOob ? kOob : b + 48, 0, 0);
        o.v4 = __builtin_amdgcn_raw_buffer_load_b32(r, rowoff == kOob ? kOob : b + 64, 0, 0);
    }
}

// First of the 8 columns (within a chunk) of product s in lane group q.
template <int FMT>
__host__ __device__ constexpr int mg_kcol(int q, int s) {
    return FMT == kQ4_K ? 64 * (q / 2 + 2 * (s >> 2)) + 32 * ((s >> 1) & 1) + 16 * (q & 1) + 8 * (s & 1)
                        : 64 * q + 8 * s;
}

// Per-chunk constants of a lane's weights: Q4_K its four sub-blocks
// 2(q/2), +1, +4, +5 (w = a*q + b with a = d*sc, b = -dmin*m); Q8_0 its two
// blocks (w = a*u - 128a, u = q + 128 read unsigned).  The decode takes each
// quant byte v as the exact fp16 value 1024 + v (exponent byte 0x64 placed by a
// byte permute, two per instruction) and forms w = a*(1024 + v) + c with
// c = b - 1024a in one mixed-precision FMA.  Q8_0: both products are exact, so w
// is the same fp32 value as a*u - 128a.  Q4_K: c is rounded once, an error of
// at most 2^-14 |a| before w is rounded to bf16.
struct MgScale {
    float a[4], c[4];
};

template <int FMT>
__device__ __forceinline__ MgScale mg_scales(const MgRaw<FMT>& r, int q) {
    MgScale s;
    if constexpr (FMT == kQ4_K) {
        const float d = half_bits_to_float(r.hdr.x);
        const float dmin = half_bits_to_float(r.hdr.x >> 16);
        const Q4KScales sc = q4k_unpack(r.hdr.y, r.hdr.z, r.hdr.w);
        const int j0 = 2 * (q >> 1);
        // sub-blocks j0, j0+1 < 4 read the low fields, j0+4, j0+5 the high ones
        const uint32_t sc_[4] = {byte_of(sc.scl, j0), byte_of(sc.scl, j0 + 1), byte_of(sc.sch, j0),
                                 byte_of(sc.sch, j0 + 1)};
        const uint32_t m_[4] = {byte_of(sc.mnl, j0), byte_of(sc.mnl, j0 + 1), byte_of(sc.mnh, j0),
                                byte_of(sc.mnh, j0 + 1)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s.a[i] = d * (float)sc_[i];
            s.c[i] = -dmin * (float)m_[i] - 1024.f * s.a[i];
        }
    } else {
        (void)q;
        s.a[0] = half_bits_to_float(r.v0.x);
        s.c[0] = -1152.f * s.a[0];
        s.a[1] = half_bits_to_float(r.v2.x >> 16);   // bytes 34-35
        s.c[1] = -1152.f * s.a[1];
        s.a[2] = s.a[3] = s.c[2] = s.c[3] = 0.f;
    }
    return s;
}

__device__ __forceinline__ uint32_t u4_at(const u32x4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The 8 weights of product s (compile-time) as a bf16 operand.
template <int FMT, int S>
__device__ __forceinline__ bf16x8 mg_decode(const MgRaw<FMT>& r, const MgScale& sc) {
    uint32_t w0, w1;
    float a, c;
    if constexpr (FMT == kQ4_K) {
        // bytes 8(S%2) .. +7 of the lane's first (S < 4) or second 16 quant
        // bytes; low nibbles for S%4 < 2, high after
        const u32x4& src = S < 4 ? r.q0 : r.q1;
        const uint32_t x0 = u4_at(src, 2 * (S & 1)), x1 = u4_at(src, 2 * (S & 1) + 1);
        constexpr int hi = (S >> 1) & 1;
        constexpr int sb = 2 * (S >> 2) + hi;
        if constexpr (!hi) {
            w0 = opaque(x0 & 0x0F0F0F0Fu);
            w1 = opaque(x1 & 0x0F0F0F0Fu);
        } else {
            w0 = opaque((x0 >> 4) & 0x0F0F0F0Fu);
            w1 = opaque((x1 >> 4) & 0x0F0F0F0Fu);
        }
        a = sc.a[sb];
        c = sc.c[sb];
    } else {
        // bytes of the lane's 68: block 2q quants at 2..33, block 2q+1 at 36..67.
        // (q ^ 0x80) read as an unsigned byte is q + 128.
        const uint32_t d[17] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w,
                                r.v2.x, r.v2.y, r.v2.z, r.v2.w, r.v3.x, r.v3.y, r.v3.z, r.v3.w,
                                r.v4};
        if constexpr (S < 4) {
            w0 = __builtin_amdgcn_alignbyte(d[2 * S + 1], d[2 * S], 2);
            w1 = __builtin_amdgcn_alignbyte(d[2 * S + 2], d[2 * S + 1], 2);
            a = sc.a[0];
            c = sc.c[0];
        } else {
            w0 = d[9 + 2 * (S - 4)];
            w1 = d[10 + 2 * (S - 4)];
            a = sc.a[1];
            c = sc.c[1];
        }
        w0 ^= 0x80808080u;
        w1 ^= 0x80808080u;
    }
    // bytes -> fp16 1024 + v, two per permute (byte 4 of the selector is 0x64)
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    constexpr uint32_t e = 0x64646464u;
    const h2 p0 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(e, w0, 0x04010400u));
    const h2 p1 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(e, w0, 0x04030402u));
    const h2 p2 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(e, w1, 0x04010400u));
    const h2 p3 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(e, w1, 0x04030402u));
    u32x4 o;
    o.x = cvt_bf16x2(__builtin_fmaf(a, (float)p0.x, c), __builtin_fmaf(a, (float)p0.y, c));
    o.y = cvt_bf16x2(__builtin_fmaf(a, (float)p1.x, c), __builtin_fmaf(a, (float)p1.y, c));
    o.z = cvt_bf16x2(__builtin_fmaf(a, (float)p2.x, c), __builtin_fmaf(a, (float)p2.y, c));
    o.w = cvt_bf16x2(__builtin_fmaf(a, (float)p3.x, c), __builtin_fmaf(a, (float)p3.y, c));
    return __builtin_bit_cast(bf16x8, o);
}

// LDS byte offset of the activation piece (product s, group g of the tile's G,
// lane l): lane indices are XOR-ed with s so that the eight pieces of one row
// written by eight neighbouring threads fall on distinct banks; a fragment
// read (64 lanes, one (s, g)) is still a permutation of one contiguous KiB.
// One chunk of a G-group tile takes 8 * G KiB.
template <int G>
__device__ __forceinline__ int mg_lds_off(int s, int g, int l) {
    return ((s * G + g) * 64 + (l ^ s)) * 16;
}

// One tile (G 16-row groups of slots, G fixed at compile time so that the
// inner loops carry no per-product branch) against 64*TPW rows of each matrix.
// NMAT = 2: gate and up (wave w holds rows 16*(w*TPW + j) .. of both
// matrices); NMAT = 1: one matrix.  NW waves per workgroup (4 and 8 measured
// the same; 4 is used).
// DENSE: a plain product (slot i = activation row i = output row i, chunk
// buffers sized for this tile's groups, optionally one of two K halves added
// onto a zeroed output); otherwise the grouped expert layout.
template <int FMT, int NMAT, int TPW, int NW, int G, bool DENSE>
__device__ __forceinline__ void mg_tile(const MgArgs& p, uint8_t* lds, int row0, int ex, int nt,
                                        int split) {
    constexpr int NT = NMAT * TPW;
    constexpr int GL = DENSE ? G : 4;        // groups in the chunk buffer layout
    constexpr int ABUF = 8 * GL * kAFrag;    // one chunk of activations
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4;

    // weights: lane rows of each column tile; rows past n read as zero
    __amdgpu_buffer_rsrc_t wr[NMAT];
    const uint32_t mbytes = (uint32_t)(p.n * p.rb);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) wr[m] = make_rsrc(p.w[m] + (int64_t)ex * p.n * p.rb, mbytes);
    uint32_t roff[TPW];
    int64_t col[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        col[j] = (int64_t)nt * (16 * TPW * NW) + 16 * (wave * TPW + j) + (lane & 15);
        roff[j] = col[j] < p.n ? (uint32_t)(col[j] * p.rb) : kOob;
    }

    // activation staging: thread pieces i = 0..PPT-1 are row tid/32 + 2*NW*i,
    // piece u = tid % 32 (product u % 8, lane group u / 8) of that row's chunk
    constexpr int PPT = 8 * G / NW;   // 16G rows x 32 pieces over 64*NW threads
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.abytes);
    const int u = tid & 31, us = u & 7, uq = u >> 3;
    const uint32_t acol = (uint32_t)(2 * mg_kcol<FMT>(uq, us));
    uint32_t asrc[PPT];   // byte offset of the row's first chunk, or kOob
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int slot = row0 + (tid >> 5) + 2 * NW * i;
        int src = slot;
        if constexpr (DENSE) {
            src = slot < p.dense_m ? slot : -1;
        } else if (p.adiv > 0) {
            const int pr = p.spair[slot];
            src = pr >= 0 ? pr / p.adiv : -1;
        }
        asrc[i] = src >= 0 ? (uint32_t)src * (uint32_t)p.k * 2u + acol : kOob;
    }
    // LDS destination of piece i: row r = tid/32 + 2*NW*i lies in group r/16 at
    // row r%16, so the offsets differ from piece 0's by constants
    const int adst0 = mg_lds_off<GL>(us, 0, (tid >> 5) + 16 * uq);
    auto adst = [&](int i) {
        return NW == 8 ? adst0 + i * kAFrag : adst0 + (i >> 1) * kAFrag + (i & 1) * 128;
    };
    u32x4 av[PPT];
    // chunks c0 .. c0 + nc - 1 of K (a dense product may split K in two)
    const int nc_all = p.k / kKC;
    const int per = DENSE ? (nc_all + p.ksplit - 1) / p.ksplit : nc_all;
    const int c0 = DENSE ? split * per : 0;
    const int nc = min(per, nc_all - c0);
    if (nc <= 0) return;
    auto load_a = [&](int cr) {
        const int c = c0 + cr;
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const uint32_t off = asrc[i] == kOob ? kOob : asrc[i] + (uint32_t)c * (kKC * 2);
            av[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
        }
    };
    auto store_a = [&](uint8_t* buf) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) *reinterpret_cast<u32x4*>(buf + adst(i)) = av[i];
    };

    MgRaw<FMT> rw[2][NT];
    auto load_w = [&](int cr, MgRaw<FMT> (&dst)[NT]) {
        const int c = c0 + cr;
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < TPW; ++j) mg_load<FMT>(wr[m], roff[j], c, q, dst[m * TPW + j]);
    };

    f32x4 acc[4][NT];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const uint8_t* buf, const MgRaw<FMT> (&cw)[NT]) {
        MgScale sc[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) sc[j] = mg_scales<FMT>(cw[j], q);
        auto step = [&](auto sc_) {
            constexpr int S = decltype(sc_)::value;
            bf16x8 af[4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                if (g < G) af[g] = *reinterpret_cast<const bf16x8*>(buf + mg_lds_off<GL>(S, g, lane));
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const bf16x8 bw = mg_decode<FMT, S>(cw[j], sc[j]);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    if (g < G)
                        acc[g][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[g], bw, acc[g][j], 0, 0, 0);
            }
            // keep each product's decode next to its matrix ops: hoisting all
            // eight decodes ahead would need more registers than two waves per
            // SIMD have
            __builtin_amdgcn_sched_barrier(0);
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
        step(std::integral_constant<int, 4>{});
        step(std::integral_constant<int, 5>{});
        step(std::integral_constant<int, 6>{});
        step(std::integral_constant<int, 7>{});
    };

    // Weights and activations run one chunk ahead (two register sets for the
    // weights, named statically: two chunks per trip; two LDS buffers for the
    // activations).  A chunk's activation loads are issued before its weight
    // loads, so storing them to LDS does not wait for the weights.  Inside the
    // loop every chunk has a successor and its loads are unconditional: a
    // branch around them would leave the wait counter unknown at the join, and
    // the compiler would then wait for the prefetch before using the current
    // chunk.  The last chunk (no successor) is peeled off.
    load_a(0);
    load_w(0, rw[0]);
    store_a(lds);
    __syncthreads();
    auto step = [&](int c, const MgRaw<FMT> (&cur)[NT], MgRaw<FMT> (&nxt)[NT]) {
        load_a(c + 1);
        load_w(c + 1, nxt);
        compute(lds + (c & 1) * ABUF, cur);
        store_a(lds + ((c + 1) & 1) * ABUF);
        __syncthreads();
    };
    int c = 0;
    for (; c + 2 < nc; c += 2) {
        step(c, rw[0], rw[1]);
        step(c + 1, rw[1], rw[0]);
    }
    if (c + 1 < nc) {
        step(c, rw[0], rw[1]);
        compute(lds + ((c + 1) & 1) * ABUF, rw[1]);
    } else {
        compute(lds + (c & 1) * ABUF, rw[0]);
    }

    // D layout: lane holds rows 4*(lane/16) + r, column lane % 16 of each product
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        if (g >= G) break;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int slot = row0 + 16 * g + 4 * q + r;
            if constexpr (NMAT == 2) {
#pragma unroll
                for (int j = 0; j < TPW; ++j) {
                    if (col[j] >= p.n) continue;
                    const float gv = acc[g][j][r], uv = acc[g][TPW + j][r];
                    const float hv = gv / (1.0f + expf(-gv)) * uv;
                    p.hout[(int64_t)slot * p.ldo + col[j]] =
                        (uint16_t)(cvt_bf16x2(hv, 0.f) & 0xFFFFu);
                }
            } else {
                const int pr = DENSE ? (slot < p.dense_m ? slot : -1) : p.spair[slot];
                if (pr < 0) continue;
#pragma unroll
                for (int j = 0; j < TPW; ++j) {
                    if (col[j] >= p.n) continue;
                    float* dst = p.dout + (int64_t)pr * p.ldo + col[j];
                    // two K halves add onto a zeroed output: 0 + a + b is the
                    // same in either order
                    if (DENSE && p.ksplit > 1) unsafeAtomicAdd(dst, acc[g][j][r]);
                    else *dst = acc[g][j][r];
                }
            }
        }
    }
}

template <int FMT, int NMAT, int TPW, int NW, bool DENSE = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void mg_kernel(const MgArgs p) {
    extern __shared__ __align__(16) uint8_t lds[];
    // blocks go to the eight XCDs round robin: XCD x takes tiles x, x+8, ...,
    // each with all its column tiles in a row, so a tile's activations are
    // fetched into one L2 only
    const int b = blockIdx.x;
    int row0, tinfo, nt, split = 0;
    if constexpr (DENSE) {
        // dense: row tiles fastest, so each column tile's row tiles run side by
        // side, then column tiles, then K halves
        const int tiles = (p.dense_m + kBM - 1) / kBM;
        const int mt = b % tiles;
        nt = (b / tiles) % p.ntn;
        split = b / tiles / p.ntn;
        row0 = mt * kBM;
        tinfo = min(4, (p.dense_m - row0 + kPad - 1) / kPad);
    } else {
        const int per = b >> 3;
        const int mt = (per / p.ntn) * 8 + (b & 7);
        nt = per % p.ntn;
        if (mt >= p.hdr[0]) return;
        row0 = p.tiles[2 * mt];
        tinfo = p.tiles[2 * mt + 1];
    }
    const int ex = tinfo >> 3;
    switch (tinfo & 7) {   // 16-row groups in this tile (1..4)
        case 1: mg_tile<FMT, NMAT, TPW, NW, 1, DENSE>(p, lds, row0, ex, nt, split); break;
        case 2: mg_tile<FMT, NMAT, TPW, NW, 2, DENSE>(p, lds, row0, ex, nt, split); break;
        case 3: mg_tile<FMT, NMAT, TPW, NW, 3, DENSE>(p, lds, row0, ex, nt, split); break;
        default: mg_tile<FMT, NMAT, TPW, NW, 4, DENSE>(p, lds, row0, ex, nt, split); break;
    }
}

template <int FMT, int NMAT, int TPW, int NW>
hipError_t launch_mg(MgArgs a, int64_t tile_bound, hipStream_t s) {
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(mg_kernel<FMT, NMAT, TPW, NW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kABuf);
        attr = true;
    }
    constexpr int rows = 16 * TPW * NW;   // rows of each matrix per workgroup
    a.ntn = (int32_t)((a.n + rows - 1) / rows);
    const int64_t mt8 = (tile_bound + 7) / 8 * 8;
    hipLaunchKernelGGL((mg_kernel<FMT, NMAT, TPW, NW>), dim3((unsigned)(mt8 * a.ntn)), dim3(64 * NW),
                       2 * kABuf, s, a);
    return hipGetLastError();
}

// A [M][K] fp32 (lda) -> bf16 [M][K], 8 values per thread; with `zero_n` > 0
// also C [M][zero_n] (ldc) := 0 for the two K halves to add onto.
__global__ __launch_bounds__(256) void mid_xbf_kernel(const float* __restrict__ a, int64_t lda,
                                                      int64_t m, int64_t k,
                                                      uint16_t* __restrict__ ab,
                                                      float* __restrict__ c, int64_t ldc,
                                                      int64_t zero_n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < m * zero_n) c[(i / zero_n) * ldc + i % zero_n] = 0.f;
    const int64_t k8 = k / 8;
    if (i >= m * k8) return;
    const int64_t row = i / k8, c8 = i % k8;
    const float4* src = reinterpret_cast<const float4*>(a + row * lda) + 2 * c8;
    const float4 v0 = src[0], v1 = src[1];
    uint4 o;
    o.x = cvt_bf16x2(v0.x, v0.y);
    o.y = cvt_bf16x2(v0.z, v0.w);
    o.z = cvt_bf16x2(v1.x, v1.y);
    o.w = cvt_bf16x2(v1.z, v1.w);
    reinterpret_cast<uint4*>(ab + row * k)[c8] = o;
}

template <int FMT>
hipError_t launch_mid_fmt(const uint8_t* w, int64_t n, int64_t k, const uint16_t* ab, int64_t m,
                          float* c, int64_t ldc, int ksplit, hipStream_t s) {
    MgArgs a{};
    a.w[0] = w;
    a.w[1] = w;
    a.n = n;
    a.rb = row_bytes_dev<FMT>(k);
    a.k = (int32_t)k;
    a.a = ab;
    a.abytes = (uint32_t)(m * k * 2);
    a.dout = c;
    a.ldo = ldc;
    a.dense_m = (int32_t)m;
    a.ksplit = ksplit;
    constexpr int NW = kMgWaves, TPW = 1;
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(mg_kernel<FMT, 1, TPW, NW, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kABuf);
        attr = true;
    }
    const int64_t ntn = (n + 16 * TPW * NW - 1) / (16 * TPW * NW);
    const int64_t tiles = (m + kBM - 1) / kBM;
    a.ntn = (int32_t)ntn;
    // two chunk buffers of the largest tile (its groups of 16 rows)
    const size_t lds = 2 * 8 * (size_t)std::min<int64_t>(4, (m + kPad - 1) / kPad) * kAFrag;
    hipLaunchKernelGGL((mg_kernel<FMT, 1, TPW, NW, true>), dim3((unsigned)(tiles * ntn * ksplit)),
                       dim3(64 * NW), lds, s, a);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const uint8_t* wg, const uint8_t* wu, const uint8_t* wd, int64_t e,
                      int64_t h, int64_t f, int64_t t, int top_k, const MgWs& m, hipStream_t s) {
    const int64_t p = t * top_k;
    const int64_t tb = moe_gemm_tile_bound(e, p), sb = moe_gemm_slot_bound(e, p);
    MgArgs a{};
    a.w[0] = wg;
    a.w[1] = wu;
    a.n = f;
    a.rb = row_bytes_dev<FMT>(h);
    a.k = (int32_t)h;
    a.a = m.xb;
    a.abytes = (uint32_t)(t * h * 2);
    a.adiv = top_k;
    a.hdr = m.hdr;
    a.tiles = m.tiles;
    a.spair = m.spair;
    a.hout = m.hb;
    a.ldo = f;
    a.ksplit = 1;
    hipError_t err = launch_mg<FMT, 2, 1, kMgWaves>(a, tb, s);
    if (err != hipSuccess) return err;
    MgArgs d{};
    d.w[0] = wd;
    d.w[1] = wd;
    d.n = h;
    d.rb = row_bytes_dev<FMT>(f);
    d.k = (int32_t)f;
    d.a = m.hb;
    d.abytes = (uint32_t)(sb * f * 2);
    d.adiv = 0;
    d.hdr = m.hdr;
    d.tiles = m.tiles;
    d.spair = m.spair;
    d.dout = m.dbuf;
    d.ldo = h;
    d.ksplit = 1;
    return launch_mg<FMT, 1, 2, kMgWaves>(d, tb, s);
}

}  // namespace

hipError_t launch_moe_gemm(int type, const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
                           int64_t e, int64_t h, int64_t f, const float* x, int64_t t,
                           const int32_t* idx, const float* probs, int top_k, float* y, void* ws,
                           hipStream_t s) {
    const int64_t p = t * top_k;
    const MgWs m = mg_carve(ws, e, t, top_k, h, f);
    hipLaunchKernelGGL(mg_group_kernel, dim3(1), dim3(1024), 0, s, idx, (int)p, (int)e, m);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t c8 = t * h / 8;
    hipLaunchKernelGGL(mg_xbf_kernel, dim3((unsigned)((c8 + 255) / 256)), dim3(256), 0, s, x, c8,
                       m.xb);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = type == kQ4_K ? launch_fmt<kQ4_K>(wg, wu, wd, e, h, f, t, top_k, m, s)
                        : launch_fmt<kQ8_0>(wg, wu, wd, e, h, f, t, top_k, m, s);
    if (err != hipSuccess) return err;
    return launch_combine(m.dbuf, idx, probs, e, h, t, top_k, y, s);
}

constexpr int64_t kMidCUs = 256;

// Products of a few tens of rows: the grouped kernel's tile (up to 64 rows of A
// in LDS, the weights decoded straight into matrix-core operands) over column
// tiles of 64 weight rows, A rounded to bf16 once.
bool gemm_mid_applies(int type, int64_t m, int64_t n, int64_t k) {
    if (type != kQ4_K && type != kQ8_0) return false;
    if (m <= 16 || m > kGemmMidRows || k % kKC != 0 || k > INT32_MAX) return false;
    if (m * k * 2 >= ((int64_t)1 << 31) || n * row_bytes(type, k) >= ((int64_t)1 << 32)) return false;
    // enough column tiles to cover the compute units
    const int64_t tiles = (m + kBM - 1) / kBM;
    return (n + 63) / 64 * tiles >= 192;
}

size_t gemm_mid_ws_bytes(int64_t m, int64_t k) { return al256((size_t)m * k * 2); }

hipError_t launch_gemm_mid(int type, const uint8_t* w, int64_t n, int64_t k, const float* a,
                           int64_t lda, int64_t m, float* c, int64_t ldc, void* ws, hipStream_t s) {
    uint16_t* ab = static_cast<uint16_t*>(ws);
    // K in two halves (added onto a zeroed C) while the workgroups of both
    // still fit the device at once: twice the loads in flight
    const int64_t wgs = (m + kBM - 1) / kBM * ((n + 63) / 64);
    const int64_t groups = std::min<int64_t>(4, (m + kPad - 1) / kPad);
    const int64_t per_cu = std::min<int64_t>(3, (160 * 1024) / (2 * 8 * groups * kAFrag));
    const int ksplit = (k / kKC >= 8 && 2 * wgs <= per_cu * kMidCUs) ? 2 : 1;
    const int64_t cnt = std::max(m * (k / 8), ksplit > 1 ? m * n : (int64_t)0);
    hipLaunchKernelGGL(mid_xbf_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s, a, lda,
                       m, k, ab, c, ldc, ksplit > 1 ? n : (int64_t)0);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return type == kQ4_K ? launch_mid_fmt<kQ4_K>(w, n, k, ab, m, c, ldc, ksplit, s)
                         : launch_mid_fmt<kQ8_0>(w, n, k, ab, m, c, ldc, ksplit, s);
}

}  // namespace ggq
