// quantize_w4: the ConvRot W4A8 weight quantiser on the GPU.
//
// ai-toolkit convrot_w4a8_quant.py, ConvRotW4A8Quantizer.quantize_ and
// _quantize_rotated_rows (with _assign_codes, grid_levels, _assign_grid):
//   0. (unless the weight is given rotated) rotate each 256-column block of a row by
//      H4^(x4) / 16 (h3-rs 0.2.0 src/weights.rs, fn hadamard): radix-4 stages in fp64,
//      exact for fp32 inputs unless a block spans more than ~29 binades, rounded once
//      to fp32;
//   1. per group of 16: gs = max(max |w|, 1e-8);
//   2. codes = nearest codebook level of fp32(w / gs): the count p of levels below the
//      value, candidates p - 1 and p (clamped), the upper one only if strictly closer,
//      distances in fp32;
//   3. twice: gs = max(fp32(num / den), 1e-8) with num = sum of fp32(w * cb[q]) and
//      den = max(sum of fp32(cb[q]^2), 1e-8), each sum accumulated in fp64 in column
//      order and rounded once to fp32; then the codes are assigned again;
//   4. s_channel = max(fp32(max over the row of |fp32(cb[q] * gs)| / 127), 1e-8);
//   5. s_rel = e4m3(fp32(gs / s_channel)), round to nearest even on the mantissa,
//      subnormals kept, magnitudes above 464 to the NaN byte;
//   6. levels = clamp(rint(fp32(cb * e4m3(s_rel))), -127, 127) (a NaN level stays NaN);
//   7. final codes = the nearest level (same rule) of fp32(w / s_channel), packed two
//      per byte, even column in the low nibble.
// The arithmetic follows the fp32 reading of the page's tensor expressions: every
// product and quotient is one IEEE fp32 operation, no contraction into FMAs.
//
// Layout: one block of 256 threads per weight row, the row taken in chunks of 4096
// columns (16 rotation blocks; slot s of 16 lanes rotates block s of the chunk, then
// every thread quantises one 16-column group).  A first pass over the chunks finds
// s_channel (a max over the whole row); a second pass repeats the rotation and the
// group fits, which are deterministic, and writes codes and scales.  Rows with at most
// 4096 columns keep the first pass's results in registers instead.
#include "w4a8_device.hpp"
#include "wquant_device.hpp"

namespace w4a8 {
namespace {

constexpr int QZ_THREADS = 256;
constexpr int QZ_CHUNK = 4096;   // columns per pass over a row

__global__ __launch_bounds__(QZ_THREADS) void quantize_kernel(const float* __restrict__ wt, int K, int rotated,
                                                              const float* __restrict__ codebook,
                                                              uint8_t* __restrict__ qpacked,
                                                              uint8_t* __restrict__ srel,
                                                              float* __restrict__ s_channel) {
    __shared__ __attribute__((aligned(16))) double tbuf[16 * 16 * QTSTRIDE];
    __shared__ float wmax[QZ_THREADS / 64];

    const int tid = threadIdx.x, slot = tid >> 4, l16 = tid & 15, lane = tid & 63;
    const int64_t row = blockIdx.x;
    const float* wrow = wt + row * K;
    float cb[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) cb[c] = codebook[c];

    // pass 1: the row's largest |cb[q] * gs|
    const int nchunk = (K + QZ_CHUNK - 1) / QZ_CHUNK;
    float w[16], lv[16];
    int q[16];
    float gs = 0.0f, rmax = 0.0f;
    for (int ch = 0; ch < nchunk; ++ch) {
        load_group(wrow, K, ch * QZ_CHUNK, rotated != 0, slot, l16, tbuf, w);
        gs = fit_group(w, cb, q, lv);
        if (ch * QZ_CHUNK + tid * 16 < K) {
#pragma unroll
            for (int k = 0; k < 16; ++k) rmax = __builtin_fmaxf(rmax, __builtin_fabsf(__fmul_rn(lv[k], gs)));
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) rmax = __builtin_fmaxf(rmax, __shfl_xor(rmax, o, 64));
    if (lane == 0) wmax[tid >> 6] = rmax;
    __syncthreads();
    rmax = wmax[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) rmax = __builtin_fmaxf(rmax, wmax[i]);   // uniform
    const float sch = __builtin_fmaxf(__fdiv_rn(rmax, 127.0f), 1e-8f);
    const double inv_sch = 1.0 / (double)sch;   // for div_by
    if (tid == 0) s_channel[row] = sch;

    // pass 2: scales, grid levels and final codes (the last chunk's fit is still held)
    const int KH = K >> 1, G = K >> 4;
    for (int ch = nchunk - 1; ch >= 0; --ch) {
        if (ch != nchunk - 1) {
            load_group(wrow, K, ch * QZ_CHUNK, rotated != 0, slot, l16, tbuf, w);
            gs = fit_group(w, cb, q, lv);
        }
        const int col = ch * QZ_CHUNK + tid * 16;
        if (col < K) {
            const uint32_t sb = f32_to_e4m3fn(__fdiv_rn(gs, sch));
            const float s = e4m3fn_to_f32(sb);
            float lvl[16];
            grid_levels16(cb, s, lvl);
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                float dummy;
                const uint32_t code = (uint32_t)nearest16(div_by(w[k], inv_sch), lvl, &dummy);
                packed[k >> 3] |= code << (4 * (k & 7));
            }
            *reinterpret_cast<uint2*>(qpacked + row * KH + (col >> 1)) = uint2{packed[0], packed[1]};
            srel[row * G + (col >> 4)] = (uint8_t)sb;
        }
    }
}

}  // namespace

hipError_t launch_quantize(const float* w, int64_t N, int K, int rotated, const float* codebook, uint8_t* qpacked,
                           uint8_t* srel, float* s_channel, hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    // rows shorter than a chunk get only the waves that hold groups of the row (K = 3072:
    // 3 waves; the fourth would fit zeros), whole waves so the lane reductions see no
    // absent lanes
    const int threads = K >= QZ_CHUNK ? QZ_THREADS : 64 * ((K / 16 + 63) / 64);
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)N), dim3((unsigned)threads), 0, stream, w, K, rotated,
                       codebook, qpacked, srel, s_channel);
    return hipGetLastError();
}

}  // namespace w4a8
