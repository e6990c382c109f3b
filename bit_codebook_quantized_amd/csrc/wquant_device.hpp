// Device helpers of the weight-side kernels (quantize_w4 and the code-only
// requantisation, fake quantisation and dequantisation): the fp64 block rotation of
// fp32 rows, the fp8 E4M3FN encoder, the nearest-level rule and the grid levels.
// ai-toolkit convrot_w4a8_quant.py (_assign_codes, grid_levels, _assign_grid) and
// h3-rs 0.2.0 src/weights.rs (fn hadamard).  Layout: a block of 256 threads is 16
// slots of 16 lanes; slot s holds rotation block s of a 4096-column chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a8_device.hpp"

namespace w4a8 {

constexpr int QTSTRIDE = 9;      // padded row of the fp64 transpose buffer (16 x 8 halves)

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

// Nearest of 16 levels ([AT] _assign_codes / _assign_grid): p = count of levels < x
// (the left insertion point for non-decreasing levels), candidates at indices p - 1 and
// p clamped to 0..15, the upper one only if strictly closer (fp32 distances).
// Returns the code; *lv receives the chosen level.
//
// nearest16 and nearest16_sorted are for non-decreasing levels (a sorted codebook and a
// non-negative scale, as in the quantiser): the candidates are then the last level below
// x and the first one not below it.  nearest16 tracks them in the same pass as the count
// (few registers: the quantiser's fit calls it three times per weight); nearest16_sorted
// finds them by binary search (fewer instructions).  nearest16_any takes the two
// candidates by index, so it follows the rule for levels in any order (stored scale bytes
// of either sign); for non-decreasing levels all three agree.
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

// Copies the 16 levels into values produced by empty asm statements.  Selects between
// table entries then act on those values; a select between two loads of the table is
// otherwise turned into one load from a selected address, which keeps the caller's level
// table in scratch memory.
__device__ __forceinline__ void levels_in_registers(const float (&lvl)[16], float (&out)[16]) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        out[c] = lvl[c];
        asm volatile("" : "+v"(out[c]));
    }
}

// A branchless binary search: five tests give p = #{c : lvl[c] < x} (pivots 7; 3 or 11;
// ...; then p itself), and, as in a search tree, the level below x is the last pivot that
// tested below it and the level not below x the last one that did not (lvl[0] / lvl[15]
// when there is none).
__device__ __forceinline__ int nearest16_sorted(float x, const float (&lv16)[16], float* lv) {
    float lvl[16];
    levels_in_registers(lv16, lvl);
    float lo = lvl[0], hi = lvl[15];
    const bool t8 = lvl[7] < x;
    lo = t8 ? lvl[7] : lo;
    hi = t8 ? hi : lvl[7];
    const float p4 = t8 ? lvl[11] : lvl[3];
    const bool t4 = p4 < x;
    lo = t4 ? p4 : lo;
    hi = t4 ? hi : p4;
    const float p2 = t8 ? (t4 ? lvl[13] : lvl[9]) : (t4 ? lvl[5] : lvl[1]);
    const bool t2 = p2 < x;
    lo = t2 ? p2 : lo;
    hi = t2 ? hi : p2;
    const float q0 = t2 ? lvl[2] : lvl[0], q1 = t2 ? lvl[6] : lvl[4], q2 = t2 ? lvl[10] : lvl[8],
                q3 = t2 ? lvl[14] : lvl[12];
    const float p1 = t8 ? (t4 ? q3 : q2) : (t4 ? q1 : q0);
    const bool t1 = p1 < x;
    lo = t1 ? p1 : lo;
    hi = t1 ? hi : p1;
    const int b = (t8 ? 8 : 0) + (t4 ? 4 : 0) + (t2 ? 2 : 0) + (t1 ? 1 : 0);   // p is b or b + 1
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = t1 ? lvl[2 * j + 1] : lvl[2 * j];
    const float f0 = t2 ? e[1] : e[0], f1 = t2 ? e[3] : e[2], f2 = t2 ? e[5] : e[4], f3 = t2 ? e[7] : e[6];
    const float pf = t8 ? (t4 ? f3 : f2) : (t4 ? f1 : f0);   // lvl[b]
    const bool t0 = pf < x;
    lo = t0 ? pf : lo;
    hi = t0 ? hi : pf;
    const int p = b + (t0 ? 1 : 0);
    const int ilo = p > 0 ? p - 1 : 0, ihi = p < 15 ? p : 15;
    const float dlo = __builtin_fabsf(__fsub_rn(x, lo)), dhi = __builtin_fabsf(__fsub_rn(x, hi));
    const bool up = dhi < dlo;
    *lv = up ? hi : lo;
    return up ? ihi : ilo;
}

__device__ __forceinline__ int nearest16_any(float x, const float (&lvl)[16], float* lv) {
    int p = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) p += lvl[c] < x ? 1 : 0;
    const int ilo = p > 0 ? p - 1 : 0, ihi = p < 15 ? p : 15;
    float L[16];
    levels_in_registers(lvl, L);
    float lo = L[0], hi = L[0];
#pragma unroll
    for (int c = 1; c < 16; ++c) {
        lo = c == ilo ? L[c] : lo;
        hi = c == ihi ? L[c] : hi;
    }
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
    double inv_gs = 1.0 / (double)gs;   // for div_by
#pragma unroll
    for (int k = 0; k < 16; ++k) q[k] = nearest16(div_by(w[k], inv_gs), cb, &lv[k]);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        double num = 0.0, den = 0.0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            num += (double)__fmul_rn(w[k], lv[k]);
            den += (double)__fmul_rn(lv[k], lv[k]);
        }
        gs = __builtin_fmaxf(__fdiv_rn((float)num, __builtin_fmaxf((float)den, tiny)), tiny);
        inv_gs = 1.0 / (double)gs;
#pragma unroll
        for (int k = 0; k < 16; ++k) q[k] = nearest16(div_by(w[k], inv_gs), cb, &lv[k]);
    }
    return gs;
}

// Rotate the 16 fp32 values a thread holds -- columns 16*l16 .. 16*l16 + 15 of rotation
// block `slot` -- in place: afterwards w[k] is the rotated value of the same column,
// rounded once to fp32.  A slot's 16 lanes sit in one wave and use only the slot's own
// 16 x QTSTRIDE doubles of tbuf (the fp64 transpose, then the fp32 re-layout of 272
// floats in the same bytes), so the exchanges are ordered within the wave and need no
// block barrier; the slot's region must not be in use by other LDS work of the wave.
static_assert((256 + 16) * sizeof(float) <= 16 * QTSTRIDE * sizeof(double), "the fp32 re-layout fits in a slot");
__device__ __forceinline__ void rotate16_in_place(float (&w)[16], int slot, int l16, double* tbuf) {
    double v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = (double)w[k];
    qradix16(v);   // digits 0, 1 of the column within the block (inside the thread)
    // transpose of the slot's 16 x 16 tile in two 16 x 8 halves, rows padded to 9 doubles
    // (conflict-free writes and reads; half the buffer of a whole tile)
    double* t = tbuf + slot * (16 * QTSTRIDE);
    double u[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) t[l16 * QTSTRIDE + i] = v[8 * h + i];
        wave_lds_sync();
        if ((l16 >> 3) == h) {
#pragma unroll
            for (int j = 0; j < 16; ++j) u[j] = t[j * QTSTRIDE + (l16 & 7)];
        }
        wave_lds_sync();
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = u[j];
    qradix16(v);   // digits 2, 3; v[i] is now column 16*i + l16 of the block
    float* f = reinterpret_cast<float*>(t);
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i * 17 + l16] = (float)(v[i] * 0.0625);
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k] = f[l16 * 17 + k];
    wave_lds_sync();
}

// Load (and unless `rotated`, rotate) the 16 columns c0 + 16*tid .. of a row into w.
// The 16 lanes of a slot call it together.  Slot s of the block covers rotation block s
// of the chunk; blocks past the row's end contribute zeros and are never stored.
__device__ __forceinline__ void load_group(const float* __restrict__ wrow, int K, int c0, bool rotated, int slot,
                                           int l16, double* tbuf, float (&w)[16]) {
    const int col = c0 + slot * 256 + l16 * 16;   // first column of this thread's 16
    const bool ok = col < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 v = ok ? reinterpret_cast<const float4*>(wrow + col)[i] : float4{0.f, 0.f, 0.f, 0.f};
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    if (!rotated) rotate16_in_place(w, slot, l16, tbuf);
}

// Grid levels of one group ([AT] grid_levels): clamp(rint(fp32(cb[c] * s)), -127, 127),
// a NaN level (NaN scale byte) staying NaN.
__device__ __forceinline__ void grid_levels16(const float (&cb)[16], float s, float (&lvl)[16]) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const float r = __builtin_rintf(__fmul_rn(cb[c], s));
        lvl[c] = r < -127.0f ? -127.0f : (r > 127.0f ? 127.0f : r);   // NaN stays NaN
    }
}

}  // namespace w4a8
