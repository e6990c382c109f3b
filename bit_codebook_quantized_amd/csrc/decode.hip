// decode_w4_to_int8: the int8 grid of a whole layer written to memory.
//
// ai-toolkit convrot_w4a8_quant.py, module docstring and unpack_w4a8_eager with
// W4A8_SAT: w8[n, k] = saturate_[-128,127](round_half_even(codebook[code] *
// e4m3(s_rel[n, k/16]))), fp32 product.  Packed byte j of a row holds the code of
// column 2j in its low nibble.
//
// The kernel streams the flattened [N, K/2] code bytes in 16-byte chunks (32
// weights, two groups of 16 sharing a scale byte each).  Because K % 32 == 0 a
// chunk never straddles a row, so chunk c reads code bytes 16c..16c+15, scale
// bytes 2c and 2c+1, and writes int8 bytes 32c..32c+31.  Bound by HBM: 16 + 2 B
// read and 32 B written per chunk (1.5625 B per weight).
#include "w4a8_device.hpp"

namespace w4a8 {
namespace {

constexpr int DEC_THREADS = 256;

__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(const uint8_t* __restrict__ qp,
                                                             const uint8_t* __restrict__ srel,
                                                             const float* __restrict__ codebook,
                                                             int64_t nchunks, int8_t* __restrict__ w8) {
    __shared__ __attribute__((aligned(16))) uint32_t lut[1024];
    build_level_table(lut, codebook, threadIdx.x, DEC_THREADS);
    __syncthreads();
    const uint4* lut4 = reinterpret_cast<const uint4*>(lut);
    const int64_t stride = (int64_t)gridDim.x * DEC_THREADS;
    for (int64_t c = (int64_t)blockIdx.x * DEC_THREADS + threadIdx.x; c < nchunks; c += stride) {
        const uint4 p = *reinterpret_cast<const uint4*>(qp + c * 16);
        const uint32_t sb = *reinterpret_cast<const uint16_t*>(srel + c * 2);
        const uint4 t0 = lut4[sb & 0xFFu], t1 = lut4[sb >> 8];
        const uint2 d0 = decode8(p.x, t0, 0x03020100u), d1 = decode8(p.y, t0, 0x03020100u);
        const uint2 d2 = decode8(p.z, t1, 0x03020100u), d3 = decode8(p.w, t1, 0x03020100u);
        uint4* o = reinterpret_cast<uint4*>(w8 + c * 32);
        o[0] = make_uint4(d0.x, d0.y, d1.x, d1.y);
        o[1] = make_uint4(d2.x, d2.y, d3.x, d3.y);
    }
}

// does nothing: the launch floor of a grid (w4a8_empty_launch)
__global__ void empty_kernel() {}

}  // namespace

hipError_t launch_empty(int blocks, int threads, hipStream_t stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(empty_kernel, dim3((unsigned)blocks), dim3((unsigned)threads), 0, stream);
    return hipGetLastError();
}

hipError_t launch_decode(const uint8_t* qp, const uint8_t* srel, const float* codebook, int64_t N, int K,
                         int8_t* w8, hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    const int64_t nchunks = N * (int64_t)(K / 32);
    // each block amortises its 4 KiB level table over >= 4 chunks per thread
    int64_t blocks = (nchunks + DEC_THREADS * 4 - 1) / (DEC_THREADS * 4);
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)blocks), dim3(DEC_THREADS), 0, stream, qp, srel, codebook,
                       nchunks, w8);
    return hipGetLastError();
}

}  // namespace w4a8
