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

namespace w4a8 {
namespace {

constexpr int QZ_THREADS = 256;
constexpr int QZ_CHUNK = 4096;   // columns per pass over a row
constexpr int QTSTRIDE = 17;     // padded row of the fp64 transpose buffer

__device__ __forceinline__ void qradix4(double& a0, double& a1, double& a2, double& a3) {
    const double s = (a0 + a1) + (a2 + a3);
    const double b0 = s - 2.0 * a3, b1 = s - 2.0 * a2, b2 = s - 2.0 * a1, b3 = s - 2.0 * a0;
    a0 = b0; a1 = b1; a2 = b2; a3 = b3;
}

__device__ __forceinline__ void qradix16(double (&v)[16]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) qradix4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
#pragma unroll
    for (int g = 0; g < 4; ++g) qradix4(v[g], v[g + 4], v[g + 8], v[g + 12]);
}

// fp32 -> OCP E4M3FN byte: round to nearest even on the mantissa, subnormals kept,
// magnitudes above 464 (half-way past the largest finite value 448) and NaN give the
// NaN byte.  Every scaling below is by a power of two, hence exact.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float x) {
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = __builtin_fabsf(x);
    if (!(a <= 464.0f)) return sign | 0x7Fu;               // NaN or too large
    if (a < 0x1p-6f) return sign | (uint32_t)(int)__builtin_rintf(a * 512.0f);
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // a = (1 + f) * 2^e
    const float f = __uint_as_float(__float_as_uint(a) - ((uint32_t)e << 23)) - 1.0f;
    int m = (int)__builtin_rintf(f * 8.0f);
    if (m == 8) { m = 0; ++e; }
    return sign | ((uint32_t)(e + 7) << 3) | (uint32_t)m;
}

// Nearest of 16 non-decreasing levels: p = count of levels < x, candidates p - 1 and
// p clamped to 0..15, the upper one only if strictly closer (fp32 distances).
// Returns the code; *lv receives the chosen level.
__device__ __forceinline__ int nearest16(float x, const float (&lvl)[16], float* lv) {
    int p = 0;
    float lo = lvl[0], hi = lvl[15];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        if (lvl[c] < x) { ++p; lo = lvl[c]; }
    }
#pragma unroll
    for (int c = 15; c >= 0; --c)
        if (!(lvl[c] < x)) hi = lvl[c];
    const int ilo = p > 0 ? p - 1 : 0, ihi = p < 15 ? p : 15;
    const float dlo = __builtin_fabsf(__fsub_rn(x, lo)), dhi = __builtin_fabsf(__fsub_rn(x, hi));
    const bool up = dhi < dlo;
    *lv = up ? hi : lo;
    return up ? ihi : ilo;
}

// Steps 1-3 on one group: returns gs; q / lv receive the codes and their levels.
__device__ __forceinline__ float fit_group(const float (&w)[16], const float (&cb)[16], int (&q)[16],
                                           float (&lv)[16]) {
    const float tiny = 1e-8f;
    float gs = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) gs = __builtin_fmaxf(gs, __builtin_fabsf(w[k]));
    gs = __builtin_fmaxf(gs, tiny);
#pragma unroll
    for (int k = 0; k < 16; ++k) q[k] = nearest16(__fdiv_rn(w[k], gs), cb, &lv[k]);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        double num = 0.0, den = 0.0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            num += (double)__fmul_rn(w[k], lv[k]);
            den += (double)__fmul_rn(lv[k], lv[k]);
        }
        gs = __builtin_fmaxf(__fdiv_rn((float)num, __builtin_fmaxf((float)den, tiny)), tiny);
#pragma unroll
        for (int k = 0; k < 16; ++k) q[k] = nearest16(__fdiv_rn(w[k], gs), cb, &lv[k]);
    }
    return gs;
}

// Rotate (or load) the 16 columns of group `gi` of the current chunk into w.  All
// threads call it (it synchronises).  Slot s of the block covers rotation block s of
// the chunk; blocks past the row's end contribute zeros and are never stored.
__device__ __forceinline__ void load_group(const float* __restrict__ wrow, int K, int c0, bool rotated, int slot,
                                           int l16, double* tbuf, float* fbuf, float (&w)[16]) {
    const int col = c0 + slot * 256 + l16 * 16;   // first column of this thread's 16
    const bool ok = col < K;
    float in[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 v = ok ? reinterpret_cast<const float4*>(wrow + col)[i] : float4{0.f, 0.f, 0.f, 0.f};
        in[4 * i] = v.x; in[4 * i + 1] = v.y; in[4 * i + 2] = v.z; in[4 * i + 3] = v.w;
    }
    if (rotated) {
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = in[k];
        return;
    }
    double v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = (double)in[k];
    qradix16(v);   // digits 0, 1 of the column within the block (inside the thread)
    double* t = tbuf + slot * (16 * QTSTRIDE);
#pragma unroll
    for (int i = 0; i < 16; ++i) t[l16 * QTSTRIDE + i] = v[i];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = t[j * QTSTRIDE + l16];
    __syncthreads();
    qradix16(v);   // digits 2, 3; v[i] is now column 16*i + l16 of the block
    float* f = fbuf + slot * (256 + 16);
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i * 17 + l16] = (float)(v[i] * 0.0625);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k] = f[l16 * 17 + k];
    __syncthreads();
}

__global__ __launch_bounds__(QZ_THREADS) void quantize_kernel(const float* __restrict__ wt, int K, int rotated,
                                                              const float* __restrict__ codebook,
                                                              uint8_t* __restrict__ qpacked,
                                                              uint8_t* __restrict__ srel,
                                                              float* __restrict__ s_channel) {
    __shared__ double tbuf[16 * 16 * QTSTRIDE];
    __shared__ float fbuf[16 * (256 + 16)];
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
        load_group(wrow, K, ch * QZ_CHUNK, rotated != 0, slot, l16, tbuf, fbuf, w);
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
    rmax = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    const float sch = __builtin_fmaxf(__fdiv_rn(rmax, 127.0f), 1e-8f);
    if (tid == 0) s_channel[row] = sch;

    // pass 2: scales, grid levels and final codes (the last chunk's fit is still held)
    const int KH = K >> 1, G = K >> 4;
    for (int ch = nchunk - 1; ch >= 0; --ch) {
        if (ch != nchunk - 1) {
            load_group(wrow, K, ch * QZ_CHUNK, rotated != 0, slot, l16, tbuf, fbuf, w);
            gs = fit_group(w, cb, q, lv);
        }
        const int col = ch * QZ_CHUNK + tid * 16;
        if (col < K) {
            const uint32_t sb = f32_to_e4m3fn(__fdiv_rn(gs, sch));
            const float s = e4m3fn_to_f32(sb);
            float lvl[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float r = __builtin_rintf(__fmul_rn(cb[c], s));
                lvl[c] = r < -127.0f ? -127.0f : (r > 127.0f ? 127.0f : r);   // NaN stays NaN
            }
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                float dummy;
                const uint32_t code = (uint32_t)nearest16(__fdiv_rn(w[k], sch), lvl, &dummy);
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
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)N), dim3(QZ_THREADS), 0, stream, w, K, rotated, codebook,
                       qpacked, srel, s_channel);
    return hipGetLastError();
}

}  // namespace w4a8
