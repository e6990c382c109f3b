// Device helpers of the activation rotation and quantisation, shared by
// rotate_quant_act and the GEMV that takes bf16 activations, so both compute the
// same values bit for bit.
//
// Rotation (h3-rs 0.2.0 src/weights.rs, fn hadamard / fn rotate_activation): each
// 256-column block of a row is multiplied by H4^(x4) / 16.  H4 = J - 2R (all-ones
// minus twice the reversal), so a radix-4 stage maps (a0..a3) to
// out_i = (a0 + a1 + a2 + a3) - 2 a_(3-i).  The stages run in fp64 on bf16 inputs,
// where the partial sums are exact, and the result is rounded once to fp32.
//
// Quantisation (ai-toolkit convrot_w4a8_quant.py, w4a8_act_quant_kernel):
// q = round_half_even(fp32(v / scale)) clamped to [-qmax, qmax], with fp32(v / scale)
// computed as fp32(v * fp64(1 / scale)) (the fp64 product is within 2^-52 of the
// quotient, which is never closer than 2^-49 to an fp32 rounding midpoint).
//
// A rotation slot is 16 lanes; 16 slots (256 threads) share a transpose buffer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a8_device.hpp"

namespace w4a8 {

// The 16 x 16 fp64 transpose of a slot goes through LDS in two halves of 8 columns, each
// a 16 x 8 tile with rows padded to 9 doubles: the 16 lanes' writes (72-byte stride) and
// reads (consecutive doubles) each cover the 32 banks once.  Half the buffer of a whole
// tile, so twice the blocks fit per compute unit.
constexpr int TSTRIDE = 9;
constexpr int ROTQ_TBUF_DOUBLES = 16 * 16 * TSTRIDE;   // one 16 x 8 tile per slot, 16 slots

// Half of one stage: out_i / 2 = s / 2 - a_(3-i).  Halving is exact in fp64 for these
// magnitudes, so four stages give the block product already divided by 16.
__device__ __forceinline__ void radix4(double& a0, double& a1, double& a2, double& a3) {
    const double s = (a0 + a1) + (a2 + a3);
    const double b0 = __builtin_fma(0.5, s, -a3), b1 = __builtin_fma(0.5, s, -a2);
    const double b2 = __builtin_fma(0.5, s, -a1), b3 = __builtin_fma(0.5, s, -a0);
    a0 = b0; a1 = b1; a2 = b2; a3 = b3;
}


// radix-16 over v[4*d1 + d0]: the stage of digit d0, then of digit d1
__device__ __forceinline__ void radix16(double (&v)[16]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) radix4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
#pragma unroll
    for (int g = 0; g < 4; ++g) radix4(v[g], v[g + 4], v[g + 8], v[g + 12]);
}

// The 16 bf16 inputs of a lane: columns 16*l16 .. 16*l16 + 15 of block `blk` of row
// `row` (two 16-byte loads).
struct RotIn {
    uint4 p0, p1;
};

__device__ __forceinline__ RotIn rot_load(const uint16_t* __restrict__ x, int64_t row, int K, int blk, int l16) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * K + (int64_t)blk * 256 + l16 * 16);
    return RotIn{src[0], src[1]};
}

// Rotate one block from its loaded inputs.  Every thread of the block must call this
// (it synchronises); threads with ok == false contribute zeros.  On return r[i] holds
// the rotated value of column 16*i + l16 of the block, rounded to fp32.
template <bool WAVE_SYNC = false>
__device__ __forceinline__ void rotate_loaded(const RotIn in, bool ok, int slot, int l16, double* tbuf,
                                              float (&r)[16]) {
    double v[16];
    const uint32_t w[8] = {in.p0.x, in.p0.y, in.p0.z, in.p0.w, in.p1.x, in.p1.y, in.p1.z, in.p1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t wi = ok ? w[i] : 0u;
        v[2 * i] = (double)__uint_as_float(wi << 16);
        v[2 * i + 1] = (double)__uint_as_float(wi & 0xFFFF0000u);
    }
    radix16(v);     // digits 0, 1 of the input column (inside the lane)
    double* t = tbuf + slot * (16 * TSTRIDE);
    double u[16];   // column l16 of the slot's tile: u[j] = lane j's v[l16]
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // columns 8h .. 8h + 7, read by lanes 8h .. 8h + 7
#pragma unroll
        for (int i = 0; i < 8; ++i) t[l16 * TSTRIDE + i] = v[8 * h + i];
        if constexpr (WAVE_SYNC) wave_lds_sync(); else __syncthreads();
        if ((l16 >> 3) == h) {
#pragma unroll
            for (int j = 0; j < 16; ++j) u[j] = t[j * TSTRIDE + (l16 & 7)];
        }
        if constexpr (WAVE_SYNC) wave_lds_sync(); else __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = u[j];
    radix16(v);     // digits 2, 3 (the lane index of the first half)
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = (float)v[i];
}

// Load and rotate block `blk` of row `row` (see rotate_loaded).
template <bool WAVE_SYNC = false>
__device__ __forceinline__ void rotate_block(const uint16_t* __restrict__ x, int64_t row, int K, int blk,
                                             bool ok, int slot, int l16, double* tbuf, float (&r)[16]) {
    RotIn in{};
    if (ok) in = rot_load(x, row, K, blk, l16);
    rotate_loaded<WAVE_SYNC>(in, ok, slot, l16, tbuf, r);
}

// Maximum over a slot's 16 lanes (one DPP row; every lane active) of values that are >= +0
// or +inf, never NaN (the output of block_absmax), taken on their bit patterns as unsigned
// integers.  The row mirror pairs lane i with i ^ 15, the half-row mirror with i ^ 7, the
// two quad permutes with i ^ 1 and i ^ 2; together they reach all 16 lanes.
// v from another lane of the same 16-lane row (a DPP source modifier, no LDS)
template <int CTRL>
__device__ __forceinline__ uint32_t row_dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float slot_max(float a) {
    uint32_t b = __float_as_uint(a);
    b = __builtin_elementwise_max(b, row_dpp_u<0x140>(b));   // row_mirror
    b = __builtin_elementwise_max(b, row_dpp_u<0x141>(b));   // row_half_mirror
    b = __builtin_elementwise_max(b, row_dpp_u<0xB1>(b));    // quad_perm [1, 0, 3, 2]
    b = __builtin_elementwise_max(b, row_dpp_u<0x4E>(b));    // quad_perm [2, 3, 0, 1]
    return __uint_as_float(b);
}

// Running maximum |v| over a lane's rotated block r.  fmaxf drops a NaN, so a block with a
// non-finite value is mapped to +inf through r[0]: a non-finite input makes every output of
// its block non-finite, and an output that overflows fp32 is +-inf, which the maximum keeps.
__device__ __forceinline__ float block_absmax(const float (&r)[16], float amax) {
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(r[i]));
    return (r[0] - r[0] != 0.0f) ? __builtin_inff() : amax;   // r - r is NaN for inf and NaN
}

// Maximum of the per-slot maxima smax[s0 .. s0 + ns - 1] (smax 16-byte aligned, at most 16
// entries).  Every entry is >= +0 or +inf, never NaN (block_absmax maps NaN to +inf), so the
// bit patterns order as unsigned integers: an integer maximum needs no NaN canonicalisation,
// and four entries come with one 16-byte read when the range allows it.
__device__ __forceinline__ float slots_max(const float* smax, int s0, int ns) {
    const uint32_t* sm = reinterpret_cast<const uint32_t*>(smax);
    uint32_t m = 0u;
    if ((s0 & 3) == 0 && (ns & 3) == 0 && s0 + ns <= 16) {
#pragma unroll
        for (int s = 0; s < 16; s += 4) {
            if (s >= ns) break;
            const uint4 v = *reinterpret_cast<const uint4*>(sm + s0 + s);
            m = __builtin_elementwise_max(m, __builtin_elementwise_max(__builtin_elementwise_max(v.x, v.y),
                                                                       __builtin_elementwise_max(v.z, v.w)));
        }
    } else {
        for (int s = s0; s < s0 + ns && s < 16; ++s) m = __builtin_elementwise_max(m, sm[s]);
    }
    return __uint_as_float(m);
}

// A row is poisoned when its maximum is not finite: its scale is NaN and all its codes 0.
__device__ __forceinline__ bool row_poisoned(float rmax) { return !(rmax <= 3.402823466e38f); }

// The row scale: amax / qmax as an IEEE fp32 division, 1.0 for an all-zero row, NaN for a
// poisoned row.
__device__ __forceinline__ float row_scale(float rmax, float qmaxf) {
    if (row_poisoned(rmax)) return __builtin_nanf("");
    return rmax > 0.0f ? rmax / qmaxf : 1.0f;
}

__device__ __forceinline__ uint8_t quant1(float v, double inv, float qmaxf) {
    // Adding 1.5 * 2^23 rounds |x| < 2^22 to an integer half-to-even (the one fp32 add),
    // and the sum's low byte is then that integer mod 256.  The clamp is applied to the
    // sum (limits 1.5 * 2^23 -+ qmax, exact), so larger |x| (a subnormal row scale) end
    // at -+qmax as well.
    constexpr float MAGIC = 12582912.0f;   // 1.5 * 2^23
    const float x = (float)((double)v * inv);
    const float y = __builtin_amdgcn_fmed3f(x + MAGIC, MAGIC - qmaxf, MAGIC + qmaxf);
    return (uint8_t)__float_as_uint(y);
}

// Quantise one rotated block held as r[i] = column 16*i + l16 and store it: the slot's
// 16 lanes transpose the codes through their own 256 bytes of LDS, qb (16-byte aligned;
// the slot's lanes are in one wave, so the accesses are ordered within the wave only).
// A poisoned row (one slot = one row) stores zeros.
__device__ __forceinline__ void quant_store(const float (&r)[16], double inv, float qmaxf, bool ok, bool poisoned,
                                            int8_t* __restrict__ xq, int64_t row, int K, int blk,
                                            int l16, uint8_t* qb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) qb[16 * i + l16] = quant1(r[i], inv, qmaxf);
    wave_lds_sync();
    uint4 out = *reinterpret_cast<const uint4*>(qb + 16 * l16);
    if (poisoned) out = make_uint4(0u, 0u, 0u, 0u);
    if (ok) *reinterpret_cast<uint4*>(xq + row * K + (int64_t)blk * 256 + 16 * l16) = out;
    wave_lds_sync();
}


}  // namespace w4a8
