// Device helpers shared by the W4A8 kernels (gfx950, wave64).
//
// Weight decode (ai-toolkit convrot_w4a8_quant.py, module docstring storage
// contract, unpack_w4a8_eager with W4A8_SAT): the int8 grid value of a weight is
// saturate_[-128,127](round_half_even(codebook[code] * e4m3(s_rel))) with the
// product in fp32.  A layer has 256 possible scale bytes and 16 codes, so every
// kernel that decodes first builds the 256 x 16 table of int8 levels in LDS
// (4 KiB) and then turns packed nibbles into int8 with byte permutes
// (v_perm_b32) against the 16-byte table row of the group's scale byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

// OCP fp8 E4M3FN byte -> fp32, exact: bias 7, 3 mantissa bits, subnormals
// m * 2^-9, no infinities, 0x7F / 0xFF are NaN.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t b) {
    const uint32_t sign = (b & 0x80u) << 24;
    const uint32_t e = (b >> 3) & 0xFu;
    const uint32_t m = b & 7u;
    if ((b & 0x7Fu) == 0x7Fu) return __uint_as_float(0x7FC00000u | sign);
    if (e == 0) return __uint_as_float(__float_as_uint((float)m * 0x1p-9f) | sign);
    return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

// One int8-grid level: fp32 product, round half to even, saturate; NaN -> 0.
__device__ __forceinline__ uint32_t grid_level(float level, float scale) {
    const float p = __fmul_rn(level, scale);
    if (p != p) return 0u;
    float r = __builtin_rintf(p);
    r = __builtin_fminf(__builtin_fmaxf(r, -128.0f), 127.0f);
    return (uint32_t)((int32_t)r) & 0xFFu;
}

// The level table (see build_level_table) from the 16 codebook values already in
// registers (uniform loads):
// nthreads must be a multiple of 4, so a thread's level quarter q is fixed.
__device__ __forceinline__ void build_level_table_regs(uint32_t* lut, const float (&cb)[16], int tid, int nthreads) {
    const int q = tid & 3;
    float c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = q == 0 ? cb[j] : q == 1 ? cb[4 + j] : q == 2 ? cb[8 + j] : cb[12 + j];
    for (int i = tid; i < 1024; i += nthreads) {
        const float s = e4m3fn_to_f32((uint32_t)(i >> 2));
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) w |= grid_level(c[j], s) << (8 * j);
        lut[i] = w;
    }
}

// Fill the LDS level table: lut[4*b + q] holds the levels of codes 4q..4q+3 for
// scale byte b, one byte each (code 4q in the low byte).  All threads of the
// block take part; the caller synchronises afterwards.
__device__ __forceinline__ void build_level_table(uint32_t* lut, const float* __restrict__ codebook,
                                                  int tid, int nthreads) {
    for (int i = tid; i < 1024; i += nthreads) {
        const int b = i >> 2, q = i & 3;
        const float s = e4m3fn_to_f32((uint32_t)b);
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) w |= grid_level(codebook[4 * q + j], s) << (8 * j);
        lut[i] = w;
    }
}

// Byte permute: result byte i = byte sel_i of the 8-byte value {hi:lo}
// (selectors 0..3 pick lo, 4..7 pick hi).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// The 8 codes of one packed dword (byte i = code 2i | code 2i+1 << 4) against the
// 16-level row t = {L0..3, L4..7, L8..11, L12..15}: .x = the levels of columns 0, 2, 4, 6,
// .y = those of columns 1, 3, 5, 7.  `id` is 0x03020100 held in a register (so the merge
// selector is one and-or; as a literal it would take an and and an or, since an
// instruction holds one literal).
__device__ __forceinline__ uint2 decode_split(uint32_t x, uint4 t, uint32_t id) {
    const uint32_t se = x & 0x07070707u;           // even codes, low 3 bits
    const uint32_t so = (x >> 4) & 0x07070707u;    // odd codes, low 3 bits
    const uint32_t lo_e = perm(t.y, t.x, se), hi_e = perm(t.w, t.z, se);
    const uint32_t lo_o = perm(t.y, t.x, so), hi_o = perm(t.w, t.z, so);
    // bit 3 of each code picks the upper half of the table: selector i or i + 4
    const uint32_t me = ((x >> 1) & 0x04040404u) | id;
    const uint32_t mo = ((x >> 5) & 0x04040404u) | id;
    return uint2{perm(hi_e, lo_e, me), perm(hi_o, lo_o, mo)};
}

// The same 8 levels in natural column order: .x = k0..k3, .y = k4..k7.
__device__ __forceinline__ uint2 decode8(uint32_t x, uint4 t, uint32_t id) {
    const uint2 s = decode_split(x, t, id);
    return uint2{perm(s.y, s.x, 0x05010400u), perm(s.y, s.x, 0x07030602u)};
}

// 0x03020100 (the identity byte selector) in a register the compiler cannot fold
__device__ __forceinline__ uint32_t opaque_identity_selector() {
    uint32_t id = 0x03020100u;
    asm volatile("" : "+v"(id));
    return id;
}

// fp32(x / s) for a divisor s > 0 used many times, with inv = fp64(1 / s): the fp64
// product x * inv is within about 2^-52 (relative) of the quotient, while a quotient of
// two fp32 numbers is either exactly an fp32 value or midpoint, or at least 2^-49
// (relative) away from every midpoint (2^-48 in the subnormal range), so rounding the
// product once to fp32 gives the IEEE quotient.  Three instructions instead of the
// ten of a correctly rounded fp32 division.
__device__ __forceinline__ float div_by(float x, double inv) { return (float)((double)x * inv); }

// Orders the LDS accesses of one wave: its LDS instructions execute in issue order, so a
// lane's later read sees another lane's earlier write of the same wave once the compiler
// keeps the program order (the fences), with no wait for the other waves.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// fp32 -> bf16 bits, round to nearest even; a NaN keeps its sign and top payload bits and
// becomes quiet ((u >> 16) | 0x40).  gfx950's v_cvt_pk_bf16_f32 does exactly this (checked
// on every special class and a million random values, NaNs included), two values at once.
typedef __bf16 w4a8_bf16x2 __attribute__((ext_vector_type(2)));
typedef float w4a8_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((w4a8_f32x2){lo, hi}, w4a8_bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)f32x2_to_bf16x2(f, 0.0f); }

// Epilogue of one output: fp32(acc) * (xs * ws) [+ bias], each op rounded on its own.
__device__ __forceinline__ float epilogue_f32(int32_t acc, float xs, float ws, const float* bias, int n) {
    float y = __fmul_rn((float)acc, __fmul_rn(xs, ws));
    if (bias) y = __fadd_rn(y, bias[n]);
    return y;
}

// SwiGLU of one gate/up pair (h3-rs 0.2.0 src/weights.rs, swiglu_interleaved):
// silu(g) * u = g / (1 + exp(-g)) * u in fp32, each operation rounded on its own.
__device__ __forceinline__ float swiglu_f32(float g, float u) {
    return __fmul_rn(__fdiv_rn(g, __fadd_rn(1.0f, expf(-g))), u);
}

__device__ __forceinline__ void store_out(void* out, int out_type, int64_t idx, int32_t acc, float y) {
    if (out_type == 0) {
        reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(y);
    } else if (out_type == 1) {
        reinterpret_cast<float*>(out)[idx] = y;
    } else {
        reinterpret_cast<int32_t*>(out)[idx] = acc;
    }
}

}  // namespace w4a8
