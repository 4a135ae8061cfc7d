// ggq_device.h -- device-side helpers shared by the gfx950 kernels.
//
// Block formats (GGUF reading; the Phobos README, "Inference", names Q8_0 and
// Q4_K_M but does not print their layout):
//   Q8_0  34 bytes / 32 weights : fp16 d | 32 x int8 q                w = d*q
//   Q4_K 144 bytes / 256 weights: fp16 d | fp16 dmin | 12 B packed 6-bit
//                                 scales+mins | 128 B of 4-bit quants
//                                 w = d*sc*q - dmin*m
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ggq {

constexpr int kQ8_0 = 8;
constexpr int kQ4_K = 12;
constexpr int kQ8Bytes = 34;
constexpr int kQ4Bytes = 144;

// Bytes of one row of K weights.
template <int FMT>
__host__ __device__ constexpr int64_t row_bytes_dev(int64_t k) {
    return FMT == kQ8_0 ? k / 32 * kQ8Bytes : k / 256 * kQ4Bytes;
}

// Hardware fp16 -> fp32 (v_cvt_f32_f16).  Exact for every finite input,
// subnormals included (fp16 denormals are preserved in the default FP mode).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    _Float16 h = __builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16 & 0xFFFFu));
    return static_cast<float>(h);
}

// Q4_K packed field -> four dwords whose bytes are the 6-bit values:
//   scl = sc[0..3], sch = sc[4..7], mnl = m[0..3], mnh = m[4..7].
// Sub-blocks 0..3 hold all six bits in bytes 0..3 (scales) / 4..7 (mins).
// Sub-blocks 4..7 hold their low four bits in the nibbles of bytes 8..11
// (scale low, min high) and their top two bits in the top bits of bytes 0..3
// (scales) / 4..7 (mins).
struct Q4KScales {
    uint32_t scl, sch, mnl, mnh;
};

__device__ __forceinline__ Q4KScales q4k_unpack(uint32_t s0, uint32_t s1, uint32_t s2) {
    Q4KScales r;
    r.scl = s0 & 0x3F3F3F3Fu;
    r.mnl = s1 & 0x3F3F3F3Fu;
    r.sch = (s2 & 0x0F0F0F0Fu) | (((s0 >> 6) & 0x03030303u) << 4);
    r.mnh = ((s2 >> 4) & 0x0F0F0F0Fu) | (((s1 >> 6) & 0x03030303u) << 4);
    return r;
}

__device__ __forceinline__ uint32_t byte_of(uint32_t v, int i) { return (v >> (8 * i)) & 0xFFu; }

// Scale and min of sub-block j (0..7).
__device__ __forceinline__ void q4k_sub(const Q4KScales& s, int j, uint32_t& sc, uint32_t& m) {
    uint32_t sv = j < 4 ? s.scl : s.sch;
    uint32_t mv = j < 4 ? s.mnl : s.mnh;
    sc = byte_of(sv, j & 3);
    m = byte_of(mv, j & 3);
}

// Signed byte i of v as float (one v_cvt_f32_i32 with a sign-extending byte select).
__device__ __forceinline__ float sbyte_f(uint32_t v, int i) {
    return static_cast<float>(static_cast<int8_t>((v >> (8 * i)) & 0xFFu));
}

// Unsigned byte i of v as float (v_cvt_f32_ubyte{i}).
__device__ __forceinline__ float ubyte_f(uint32_t v, int i) {
    return static_cast<float>((v >> (8 * i)) & 0xFFu);
}

// The value unchanged, but opaque to the optimiser.  After a nibble mask
// (q & 0x0F0F0F0F) the compiler otherwise uses the known zero bits to turn each
// byte conversion into a bit-field extract plus v_cvt_f32_ubyte0, one more
// instruction per weight than v_cvt_f32_ubyte{0,1,2,3} on the masked word.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of data that is read exactly once (weights): non-temporal, so it
// does not evict the activations and partial results from the caches.
__device__ __forceinline__ uint4 load_once16(const void* p) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw buffer descriptor over [base, base + bytes): loads at offsets >= bytes
// return zero, which is how tile and chunk edges are handled without branches.
// Word 3 is the CDNA raw-buffer setting (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// The same for a base and size that are equal across the wave but that the
// compiler cannot prove so (values carried through loops and LDS): it takes
// lane 0's, so the descriptor sits in scalar registers.  A descriptor in
// vector registers makes every load through it a loop over distinct lanes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base,
                                                                    uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                     __builtin_amdgcn_readfirstlane(bytes));
}

constexpr uint32_t kOob = 0xFFFFFFF0u;  // an offset past any descriptor's range

// 16-byte buffer load; `nt` marks data read exactly once (non-temporal).
template <bool NT>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace ggq
