// dequant.hip -- quant_dequantize: materialise fp32 weights from Q8_0 / Q4_K blocks.
//
// The decode itself is exact (see the block definitions in ggq_device.h): Q8_0
// d*q and Q4_K d*sc*q, dmin*m are exact fp32 products, and the Q4_K difference
// d*sc*q - dmin*m is rounded once, whether or not the compiler contracts it to an
// FMA.  One thread decodes one 32-weight run (a Q8_0 block or a Q4_K sub-block).
#include "ggq_device.h"
#include "ggq_launch.h"

namespace ggq {

__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const uint8_t* __restrict__ w,
                                                           int64_t nblocks,
                                                           float* __restrict__ out) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const uint8_t* blk = w + b * kQ8Bytes;
    // The block start is only 2-byte aligned: read it as 17 halfwords.
    const uint16_t* h = reinterpret_cast<const uint16_t*>(blk);
    float d = half_bits_to_float(h[0]);
    float4* o = reinterpret_cast<float4*>(out + b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t v = (uint32_t)h[1 + 2 * i] | ((uint32_t)h[2 + 2 * i] << 16);
        o[i] = make_float4(d * sbyte_f(v, 0), d * sbyte_f(v, 1), d * sbyte_f(v, 2),
                           d * sbyte_f(v, 3));
    }
}

// Thread = (super-block, sub-block j).  Sub-block j uses quant bytes
// qs[32*(j/2) .. +31], low nibbles for even j, high nibbles for odd j.
__global__ __launch_bounds__(256) void dequant_q4_k_kernel(const uint8_t* __restrict__ w,
                                                           int64_t nsub,
                                                           float* __restrict__ out) {
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nsub) return;
    int64_t sbi = t >> 3;
    int j = (int)(t & 7);
    const uint8_t* sb = w + sbi * kQ4Bytes;
    const uint32_t* s32 = reinterpret_cast<const uint32_t*>(sb);  // 16-byte aligned
    uint32_t h0 = s32[0];
    float d = half_bits_to_float(h0);
    float dmin = half_bits_to_float(h0 >> 16);
    Q4KScales sc = q4k_unpack(s32[1], s32[2], s32[3]);
    uint32_t scj, mj;
    q4k_sub(sc, j, scj, mj);
    const uint32_t* q32 = reinterpret_cast<const uint32_t*>(sb + 16 + 32 * (j >> 1));
    int sh = (j & 1) ? 4 : 0;
    float* o = out + t * 32;
    float dm = dmin * (float)mj;  // exact: 11-bit * 6-bit significands
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t v = (q32[i] >> sh) & 0x0F0F0F0Fu;
        float4 r;
        // d * (sc*q): sc*q < 1024 is an exact integer, the product is exact,
        // and the subtraction rounds once.
        r.x = d * (float)(scj * byte_of(v, 0)) - dm;
        r.y = d * (float)(scj * byte_of(v, 1)) - dm;
        r.z = d * (float)(scj * byte_of(v, 2)) - dm;
        r.w = d * (float)(scj * byte_of(v, 3)) - dm;
        reinterpret_cast<float4*>(o)[i] = r;
    }
}

hipError_t launch_dequant(int type, const uint8_t* w, int64_t n, int64_t k, float* out,
                          hipStream_t s) {
    if (type == kQ8_0) {
        int64_t nb = n * (k / 32);
        int64_t grid = (nb + 255) / 256;
        hipLaunchKernelGGL(dequant_q8_0_kernel, dim3((unsigned)grid), dim3(256), 0, s, w, nb, out);
    } else {
        int64_t ns = n * (k / 256) * 8;
        int64_t grid = (ns + 255) / 256;
        hipLaunchKernelGGL(dequant_q4_k_kernel, dim3((unsigned)grid), dim3(256), 0, s, w, ns, out);
    }
    return hipGetLastError();
}

}  // namespace ggq
