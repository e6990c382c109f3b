// rotate_quant_act: block-256 regular-Hadamard rotation of bf16 activation rows
// followed by per-row symmetric int8 quantisation.
//
// Rotation (h3-rs 0.2.0 src/weights.rs, fn hadamard / fn rotate_activation): each
// 256-column block of a row is multiplied by H4^(x4) / 16, where H4 is the 4x4
// regular Hadamard matrix (ones, minus ones on the anti-diagonal).  H4 = J - 2R
// (all-ones minus twice the reversal), so one radix-4 stage maps (a0..a3) to
// out_i = (a0 + a1 + a2 + a3) - 2 a_(3-i); four stages, one per base-4 digit of
// the column index, give the whole block.
//
// Precision: inputs are bf16 (8 significant bits).  The stages run in fp64.  After
// stage t a value is a sum of 4^t inputs halved t times: below 2^(E + 1 + t) in
// magnitude (E the exponent of the block's largest input) and a multiple of 2^(L - t)
// (L the exponent of the lowest set significand bit among its non-zero inputs), so
// every partial sum is exact while E - L <= 44 (for bf16: every non-zero magnitude
// within 2^37 of the block's largest).  The result is then the exact block product,
// rounded once to fp32.  This is the value the quantiser sees.
//
// Non-finite values: a row any of whose rotated values is not finite (an inf or NaN
// input, or a block whose product overflows fp32) gets scale NaN and all codes 0.
//
// Quantisation (ai-toolkit convrot_w4a8_quant.py, w4a8_act_quant_kernel): amax =
// max |v| over the row, scale = amax / qmax in fp32 (1.0 when amax is 0),
// q = round_half_even(fp32(v / scale)) clamped to [-qmax, qmax].  fp32(v / scale)
// is computed as fp32(v * fp64(1 / scale)): the fp64 product is within 2^-52
// relative of v / scale, while a quotient of two fp32 numbers is never an fp32
// rounding midpoint and sits at least 2^-49 (relative) away from one, so the
// rounding to fp32 is the IEEE quotient's.
//
// Layout: a block of 256 threads is 16 "slots" of 16 lanes; a slot rotates one
// 256-column block.  Lane j loads columns 16j..16j+15 (two 16-byte loads), runs
// the two stages of the low digits in registers, exchanges the 16 x 16 fp64
// intermediate through LDS (transpose), runs the two stages of the high digits,
// and ends with outputs 16i + j (i = 0..15).  Rows with K <= 4096 share a block
// (16 / (K/256) rows per block); longer rows take 16 columns-blocks per pass and
// keep up to CH passes of rotated values in registers between the absmax and the
// quantisation, or recompute them (CH == 0) for very long rows.
#include "w4a8_device.hpp"
#include "rotq_device.hpp"

namespace w4a8 {
namespace {

constexpr int RQ_THREADS = 256;

template <int CH>
__global__ __launch_bounds__(RQ_THREADS) void rotate_quant_kernel(const uint16_t* __restrict__ x, int64_t M, int K,
                                                                  int qmax, int8_t* __restrict__ xq,
                                                                  float* __restrict__ xs) {
    // A slot's 16 lanes sit in one wave, and the slot uses only its own part of tbuf (the
    // fp64 transposes, then the code transpose in its first 256 bytes), so those exchanges
    // are ordered within the wave, with no block barrier; the row maximum is the one
    // exchange between waves.  At 18.5 KB of LDS, 8 blocks share a CU.
    __shared__ __attribute__((aligned(16))) double tbuf[16 * 16 * TSTRIDE];
    static_assert(256 <= 16 * TSTRIDE * sizeof(double), "a slot's code transpose fits in its part of tbuf");
    __shared__ __attribute__((aligned(16))) float smax[16];

    const int tid = threadIdx.x, slot = tid >> 4, l16 = tid & 15;
    uint8_t* const qb = reinterpret_cast<uint8_t*>(tbuf + slot * 16 * TSTRIDE);
    const int nb = K >> 8;
    int rows_per_wg, row_local, blk0, nch;
    if (nb <= 16) {
        // quotients of integers below 17 by nb <= 16 from the approximate reciprocal: the
        // exact quotient plus 1/2 is at least 1/32 away from an integer, far above its error
        const float rn = __builtin_amdgcn_rcpf((float)nb);
        rows_per_wg = (int)(16.5f * rn); row_local = (int)(((float)slot + 0.5f) * rn);
        blk0 = slot - row_local * nb; nch = 1;
    } else {
        rows_per_wg = 1; row_local = 0; blk0 = slot; nch = (nb + 15) >> 4;
    }
    const int64_t row = (int64_t)blockIdx.x * rows_per_wg + row_local;
    const bool row_ok = row_local < rows_per_wg && row < M;
    const float qmaxf = (float)qmax;

    constexpr int KEEP = CH > 0 ? CH : 1;
    float keep[KEEP][16];
    float amax = 0.0f;
    if (CH > 0) {
#pragma unroll
        for (int c = 0; c < KEEP; ++c) {
            if (c < nch) {
                const int blk = blk0 + 16 * c;
                rotate_block<true>(x, row, K, blk, row_ok && blk < nb, slot, l16, tbuf, keep[c]);
                amax = block_absmax(keep[c], amax);
            }
        }
    } else {
        for (int c = 0; c < nch; ++c) {
            const int blk = blk0 + 16 * c;
            float r[16];
            rotate_block<true>(x, row, K, blk, row_ok && blk < nb, slot, l16, tbuf, r);
            amax = block_absmax(r, amax);
        }
    }

    // row absmax: over the slot's 16 lanes, then over the row's slots
    amax = slot_max(amax);
    if (l16 == 0) smax[slot] = amax;
    __syncthreads();
    const float rmax = nb <= 16 ? slots_max(smax, row_local * nb, nb) : slots_max(smax, 0, 16);
    const float scale = row_scale(rmax, qmaxf);
    const bool poisoned = row_poisoned(rmax);
    const double inv = poisoned ? 0.0 : 1.0 / (double)scale;
    if (row_ok && l16 == 0 && blk0 == 0) xs[row] = scale;

    if (CH > 0) {
#pragma unroll
        for (int c = 0; c < KEEP; ++c) {
            if (c < nch) {
                const int blk = blk0 + 16 * c;
                quant_store(keep[c], inv, qmaxf, row_ok && blk < nb, poisoned, xq, row, K, blk, l16, qb);
            }
        }
    } else {
        for (int c = 0; c < nch; ++c) {
            const int blk = blk0 + 16 * c;
            float r[16];
            rotate_block<true>(x, row, K, blk, row_ok && blk < nb, slot, l16, tbuf, r);
            quant_store(r, inv, qmaxf, row_ok && blk < nb, poisoned, xq, row, K, blk, l16, qb);
        }
    }
}

}  // namespace

// Rows per block and the register-kept pass count follow K; grid = ceil(M / rows).
hipError_t launch_rotate_quant(const uint16_t* x, int64_t M, int K, int qmax, int8_t* xq, float* xs,
                               hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    const int nb = K >> 8;
    const int rows_per_wg = nb <= 16 ? 16 / nb : 1;
    const int nch = nb <= 16 ? 1 : (nb + 15) / 16;
    const int64_t grid = (M + rows_per_wg - 1) / rows_per_wg;
    // only the slots that hold a block of a row: when nb does not divide 16 (K = 3072:
    // 12 slots) the rest would run the whole rotation on zeros
    const int threads = nb <= 16 ? 16 * nb * rows_per_wg : RQ_THREADS;
    const dim3 g((unsigned)grid), b((unsigned)threads);
    if (nch <= 1) hipLaunchKernelGGL(rotate_quant_kernel<1>, g, b, 0, stream, x, M, K, qmax, xq, xs);
    else if (nch <= 2) hipLaunchKernelGGL(rotate_quant_kernel<2>, g, b, 0, stream, x, M, K, qmax, xq, xs);
    else if (nch <= 3) hipLaunchKernelGGL(rotate_quant_kernel<3>, g, b, 0, stream, x, M, K, qmax, xq, xs);
    else if (nch <= 4) hipLaunchKernelGGL(rotate_quant_kernel<4>, g, b, 0, stream, x, M, K, qmax, xq, xs);
    else if (nch <= 8) hipLaunchKernelGGL(rotate_quant_kernel<8>, g, b, 0, stream, x, M, K, qmax, xq, xs);
    else hipLaunchKernelGGL(rotate_quant_kernel<0>, g, b, 0, stream, x, M, K, qmax, xq, xs);
    return hipGetLastError();
}

}  // namespace w4a8
