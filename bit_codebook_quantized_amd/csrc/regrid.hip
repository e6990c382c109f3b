// Weight-side kernels of the training path, on a layer's stored scales (ai-toolkit
// convrot_w4a8_quant.py, ConvRotW4A8Quantizer):
//
//   requantize_codes  -- requantize_codes_: new codes for an fp32 weight on the stored
//                        group scales, channel scales and codebook.  The weight is
//                        rotated (fp64 block rotation, rounded once to fp32) unless given
//                        rotated; target = fp32(w_rot / s_channel); the code is the
//                        nearest grid level (_assign_grid), or with uniform draws u the
//                        stochastic choice between the two bracketing levels: with p the
//                        count of levels below the target and lo = clamp(p - 1, 0, 14),
//                        thr = fp32(fp32(u * fp32(lv[lo+1] - lv[lo])) + lv[lo]) and the
//                        code is lo + (target > thr).
//   fake_quant        -- fake_quant_rotated_weight: the nearest grid level of
//                        fp32(w_rot / s_channel) times s_channel (fp32).
//   dequantize        -- dequantize_w4a8: fp32(w8 * s_channel), rotated back to the plain
//                        basis (the fp64 block sum of these terms is exact; rounded once).
//   lora_merge        -- h3-rs src/weights.rs QLinear::merge_loras for this format: the
//                        dequantised plain-basis weight plus one adapter's delta
//                        fp32(scale * sum_r B[n, r] * A[r, k]) (fp64 products and sums in
//                        r order, no fused multiply-add), added in fp32; the result goes
//                        back through quantize_w4.
//
// Layout: a block of 256 threads covers one 4096-column chunk of one row (grid =
// rows x chunks); thread t holds the 16 columns of group t of the chunk, which is the
// layout of the rotation helpers (slot t / 16 rotates block t / 16 of the chunk).
// Fake quantisation needs no rotation and uses the same mapping.
#include "w4a8_device.hpp"
#include "wquant_device.hpp"

namespace w4a8 {
namespace {

constexpr int RG_THREADS = 256;
constexpr int RG_CHUNK = 4096;
// threads per block of the nearest-level requantisation: a row shorter than a chunk gets
// only the whole waves that hold its groups (K = 3072: 3 waves; the rest would rotate
// zeros).  The stochastic form, which also reads the draws, measured slower that way.
inline int rg_threads(int K) { return K >= RG_CHUNK ? RG_THREADS : 64 * ((K / 16 + 63) / 64); }

// Stochastic bracket choice ([AT] _assign_grid, stochastic branch) among 16
// non-decreasing levels; comparisons with a NaN level are false.
// The grid levels of a group are non-decreasing when the codebook is sorted ascending and
// the group scale is not negative (NaN fails both tests).
__device__ __forceinline__ bool levels_ascend(const float (&cb)[16], float s) {
    bool a = s >= 0.0f;
#pragma unroll
    for (int c = 0; c < 15; ++c) a = a && cb[c] <= cb[c + 1];
    return a;
}

// The 16 grid levels of one scale as a packed byte row (level c in byte c % 4 of word
// c / 4), the operand of decode8.
__device__ __forceinline__ uint4 level_row(const float (&cb)[16], float s) {
    uint32_t tw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        tw[j] = grid_level(cb[4 * j], s) | grid_level(cb[4 * j + 1], s) << 8 | grid_level(cb[4 * j + 2], s) << 16 |
                grid_level(cb[4 * j + 3], s) << 24;
    return uint4{tw[0], tw[1], tw[2], tw[3]};
}

// One group's 16 weights (codes q, 8 bytes) as fp32(level * s_channel): a byte-permute
// decode against the level row, no per-weight codebook reads.
__device__ __forceinline__ void decode_group_f32(uint2 q, uint4 t, float sch, float (&w)[16]) {
    const uint2 d0 = decode8(q.x, t, 0x03020100u), d1 = decode8(q.y, t, 0x03020100u);
    const uint32_t d[4] = {d0.x, d0.y, d1.x, d1.y};
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k] = __fmul_rn((float)(int8_t)(uint8_t)(d[k >> 2] >> (8 * (k & 3))), sch);
}

__device__ __forceinline__ uint32_t stochastic16(float x, float u, const float (&lvl)[16]) {
    int p = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) p += lvl[c] < x ? 1 : 0;
    const int lo = p < 1 ? 0 : (p > 15 ? 14 : p - 1);
    float l0 = lvl[0], l1 = lvl[1];
#pragma unroll
    for (int c = 1; c < 15; ++c) {
        l0 = lo == c ? lvl[c] : l0;
        l1 = lo == c ? lvl[c + 1] : l1;
    }
    const float thr = __fadd_rn(__fmul_rn(u, __fsub_rn(l1, l0)), l0);
    return (uint32_t)(lo + (x > thr ? 1 : 0));
}

__device__ __forceinline__ void load16(const float* __restrict__ p, float (&v)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 f = reinterpret_cast<const float4*>(p)[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
}

__device__ __forceinline__ void store16(float* __restrict__ p, const float (&v)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<float4*>(p)[i] = float4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
}

// Store a wave's 64 x 16 values, lane l holding elements 16l .. 16l + 15 of 1024 consecutive
// floats at dst (elements at or past `valid` are not stored; valid is a multiple of 4).
// The values are re-laid out through the wave's 4 KiB of LDS `buf` so that each store
// instruction writes 1 KiB, not 16-byte pieces 64 bytes apart; chunk j of lane l sits at
// chunk position j ^ ((l >> 2) & 3) of its 64 bytes, which keeps the writes and the reads
// conflict-free.  buf is the wave's own (the 4 rotation slots of the wave, which it has
// finished with), so the exchange is ordered within the wave: no block barrier.
__device__ __forceinline__ void wave_store1024(float* __restrict__ dst, int64_t valid, const float (&w)[16],
                                               float* buf) {
    const int lane = threadIdx.x & 63;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(buf + 16 * lane + 4 * (j ^ ((lane >> 2) & 3))) =
            float4{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int src = 16 * i + (lane >> 2), j = lane & 3;   // the lane and chunk that hold it
        const float4 v = *reinterpret_cast<const float4*>(buf + 16 * src + 4 * (j ^ ((src >> 2) & 3)));
        if (256 * i + 4 * lane < valid) *reinterpret_cast<float4*>(dst + 256 * i + 4 * lane) = v;
    }
    wave_lds_sync();
}

// The wave's part of a rotation buffer (its 4 slots, 4608 bytes, 16-byte aligned): the
// staging buffer of wave_store1024.
__device__ __forceinline__ float* wave_region(double* tbuf) {
    return reinterpret_cast<float*>(tbuf + (threadIdx.x >> 6) * 4 * 16 * QTSTRIDE);
}
static_assert(1024 * sizeof(float) <= 4 * 16 * QTSTRIDE * sizeof(double), "a wave's staging fits in its slots");

// STOCH: stochastic rounding with the uniform draws u, else the nearest level (one path per
// instantiation: with both in one kernel the compiler moved the level table to scratch).
template <bool STOCH>
__global__ __launch_bounds__(RG_THREADS) void requant_kernel(const float* __restrict__ wt, int K, int nchunk,
                                                             int rotated, const float* __restrict__ codebook,
                                                             const uint8_t* __restrict__ srel,
                                                             const float* __restrict__ s_channel,
                                                             const float* __restrict__ u,
                                                             uint8_t* __restrict__ qpacked) {
    __shared__ __attribute__((aligned(16))) double tbuf[16 * 16 * QTSTRIDE];
    const int tid = threadIdx.x, slot = tid >> 4, l16 = tid & 15;
    const int64_t row = blockIdx.x / nchunk;
    const int c0 = (blockIdx.x - (int)(row * nchunk)) * RG_CHUNK;
    float w[16];
    load_group(wt + row * K, K, c0, rotated != 0, slot, l16, tbuf, w);   // block-uniform
    const int col = c0 + tid * 16;
    if (col >= K) return;
    float cb[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) cb[c] = codebook[c];
    const float sch = s_channel[row];
    const double inv_sch = 1.0 / (double)sch;   // for div_by
    float lvl[16];
    const float s = e4m3fn_to_f32(srel[row * (K >> 4) + (col >> 4)]);
    grid_levels16(cb, s, lvl);
    float r[16];
    if constexpr (STOCH) load16(u + row * K + col, r);
    const bool asc = !STOCH && levels_ascend(cb, s);
    uint32_t packed[2] = {0u, 0u};
    if constexpr (STOCH) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            packed[k >> 3] |= stochastic16(div_by(w[k], inv_sch), r[k], lvl) << (4 * (k & 7));
    } else if (asc) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float dummy;
            packed[k >> 3] |= (uint32_t)nearest16_sorted(div_by(w[k], inv_sch), lvl, &dummy) << (4 * (k & 7));
        }
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float dummy;
            packed[k >> 3] |= (uint32_t)nearest16_any(div_by(w[k], inv_sch), lvl, &dummy) << (4 * (k & 7));
        }
    }
    *reinterpret_cast<uint2*>(qpacked + row * (K >> 1) + (col >> 1)) = uint2{packed[0], packed[1]};
}

// One thread per 16-column group, no rotation.
__global__ __launch_bounds__(RG_THREADS) void fake_quant_kernel(const float* __restrict__ w_rot, int64_t groups,
                                                                int K, const float* __restrict__ codebook,
                                                                const uint8_t* __restrict__ srel,
                                                                const float* __restrict__ s_channel,
                                                                float* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * RG_THREADS + threadIdx.x;
    if (g >= groups) return;
    const int64_t row = g / (K >> 4);
    float cb[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) cb[c] = codebook[c];
    float lvl[16];
    const float s = e4m3fn_to_f32(srel[g]);
    grid_levels16(cb, s, lvl);
    const bool asc = levels_ascend(cb, s);
    const float sch = s_channel[row];
    const double inv_sch = 1.0 / (double)sch;   // for div_by
    float w[16], y[16];
    load16(w_rot + g * 16, w);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        float lv;
        const float t = div_by(w[k], inv_sch);
        (void)(asc ? nearest16_sorted(t, lvl, &lv) : nearest16_any(t, lvl, &lv));
        y[k] = __fmul_rn(lv, sch);
    }
    store16(out + g * 16, y);   // (a re-layout through LDS for whole-KiB stores measured no faster here)
}

__global__ __launch_bounds__(RG_THREADS) void dequant_kernel(const uint8_t* __restrict__ qpacked,
                                                             const uint8_t* __restrict__ srel,
                                                             const float* __restrict__ codebook,
                                                             const float* __restrict__ s_channel, int K, int nchunk,
                                                             int rotate_back, float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) double tbuf[16 * 16 * QTSTRIDE];
    const int tid = threadIdx.x, slot = tid >> 4, l16 = tid & 15;
    const int64_t row = blockIdx.x / nchunk;
    const int c0 = (blockIdx.x - (int)(row * nchunk)) * RG_CHUNK;
    const int col = c0 + tid * 16;
    const bool ok = col < K;
    float cb[16];   // uniform loads
#pragma unroll
    for (int c = 0; c < 16; ++c) cb[c] = codebook[c];
    float w[16];
    if (ok) {
        const float s = e4m3fn_to_f32(srel[row * (K >> 4) + (col >> 4)]);
        const float sch = s_channel[row];
        const uint2 q = *reinterpret_cast<const uint2*>(qpacked + row * (K >> 1) + (col >> 1));
        decode_group_f32(q, level_row(cb, s), sch, w);
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = 0.0f;
    }
    if (rotate_back) rotate16_in_place(w, slot, l16, tbuf);   // block-uniform
    const int wcol = c0 + (tid >> 6) * 1024;   // the wave's first column
    wave_store1024(out + row * K + wcol, K - wcol, w, wave_region(tbuf));
}

// The dequantised, rotated-back weight plus a low-rank delta (one block per row chunk).
// LoRA merge: a block of LM_THREADS threads (LM_THREADS / 16 rotation blocks, LM_CHUNK
// columns) merges LM_ROWS rows, so every A element it loads serves LM_ROWS rows (A is read
// N / LM_ROWS times in all, from L2).  Thread t holds the deltas of columns
// c0 + 16 t .. c0 + 16 t + 15 of each row in fp64; the B entries are block-uniform.
constexpr int LM_THREADS = 128, LM_ROWS = 4, LM_CHUNK = LM_THREADS * 16;
static_assert(LM_THREADS % 64 == 0 && RG_THREADS % 64 == 0, "whole waves: each has its 4 rotation slots");

__global__ __launch_bounds__(LM_THREADS) void lora_merge_kernel(const uint8_t* __restrict__ qpacked,
                                                                const uint8_t* __restrict__ srel,
                                                                const float* __restrict__ codebook,
                                                                const float* __restrict__ s_channel, int64_t N,
                                                                int K, int nchunk, const float* __restrict__ lora_a,
                                                                const float* __restrict__ lora_b, int rank,
                                                                float scale, float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) double tbuf[(LM_THREADS / 16) * 16 * QTSTRIDE];
    const int tid = threadIdx.x, slot = tid >> 4, l16 = tid & 15;
    const int64_t row0 = (int64_t)(blockIdx.x / nchunk) * LM_ROWS;
    const int c0 = (int)(blockIdx.x % nchunk) * LM_CHUNK;
    const int col = c0 + tid * 16;
    const bool ok = col < K;

    // delta[row][k] = sum over r, in order, of fp64(b[row][r]) * fp64(a[r][k]), each product
    // and sum rounded in fp64
    double d[LM_ROWS][16];
#pragma unroll
    for (int i = 0; i < LM_ROWS; ++i)
#pragma unroll
        for (int k = 0; k < 16; ++k) d[i][k] = 0.0;
    // B entries are block-uniform; an opaque per-lane zero offset makes their loads vector
    // loads, counted in order with the A loads (scalar loads would each be waited for in turn)
    int zero = 0;
    asm volatile("" : "+v"(zero));
    const float* brow[LM_ROWS];
#pragma unroll
    for (int i = 0; i < LM_ROWS; ++i) brow[i] = lora_b + (row0 + i < N ? row0 + i : N - 1) * rank + zero;
    // A loads are unconditional (lanes past the row end read its last 16 columns, and their
    // deltas are never stored) and alternate between two named buffers, so the loads of
    // r + 1 are in flight while r is accumulated
    const float* acol = lora_a + (ok ? col : K - 16);
    struct Term {
        float a[16], b[LM_ROWS];
    };
    auto load_term = [&](Term& t, int r) __attribute__((always_inline)) {
        load16(acol + (int64_t)r * K, t.a);
#pragma unroll
        for (int i = 0; i < LM_ROWS; ++i) t.b[i] = brow[i][r];
    };
    auto accumulate = [&](const Term& t) __attribute__((always_inline)) {
        double ad[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) ad[k] = (double)t.a[k];
#pragma unroll
        for (int i = 0; i < LM_ROWS; ++i) {
            const double b = (double)t.b[i];
#pragma unroll
            for (int k = 0; k < 16; ++k) d[i][k] = __dadd_rn(d[i][k], __dmul_rn(b, ad[k]));
        }
    };
    Term tA, tB;
    int r = 0;
    if (rank > 0) {
        load_term(tA, 0);
        for (; r + 1 < rank; r += 2) {
            load_term(tB, r + 1);
            accumulate(tA);
            load_term(tA, r + 2 < rank ? r + 2 : rank - 1);   // past the end: a reload
            accumulate(tB);
        }
        if (r < rank) accumulate(tA);
    }

    const double sc = (double)scale;
    float cb[16];   // uniform loads
#pragma unroll
    for (int c = 0; c < 16; ++c) cb[c] = codebook[c];
#pragma unroll
    for (int i = 0; i < LM_ROWS; ++i) {
        const int64_t row = row0 + i;
        if (row >= N) break;   // block-uniform
        float w[16];
        if (ok) {
            const float s = e4m3fn_to_f32(srel[row * (K >> 4) + (col >> 4)]);
            const float sch = s_channel[row];
            const uint2 q = *reinterpret_cast<const uint2*>(qpacked + row * (K >> 1) + (col >> 1));
            decode_group_f32(q, level_row(cb, s), sch, w);
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) w[k] = 0.0f;
        }
        rotate16_in_place(w, slot, l16, tbuf);   // all threads: back to the plain basis
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = __fadd_rn(w[k], (float)__dmul_rn(d[i][k], sc));
        const int wcol = c0 + (tid >> 6) * 1024;   // the wave's first column
        wave_store1024(out + row * K + wcol, K - wcol, w, wave_region(tbuf));
    }
}

}  // namespace

hipError_t launch_lora_merge(const uint8_t* qpacked, const uint8_t* srel, const float* codebook,
                             const float* s_channel, int64_t N, int K, const float* lora_a, const float* lora_b,
                             int rank, float scale, float* out, hipStream_t stream) {
    (void)hipGetLastError();
    const int nchunk = (K + LM_CHUNK - 1) / LM_CHUNK;
    const int64_t blocks = (N + LM_ROWS - 1) / LM_ROWS * nchunk;
    hipLaunchKernelGGL(lora_merge_kernel, dim3((unsigned)blocks), dim3(LM_THREADS), 0, stream, qpacked, srel,
                       codebook, s_channel, N, K, nchunk, lora_a, lora_b, rank, scale, out);
    return hipGetLastError();
}

hipError_t launch_requantize(const float* w, int64_t N, int K, int rotated, const float* codebook,
                             const uint8_t* srel, const float* s_channel, const float* u, uint8_t* qpacked,
                             hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    const int nchunk = (K + RG_CHUNK - 1) / RG_CHUNK;
    if (u)
        hipLaunchKernelGGL(requant_kernel<true>, dim3((unsigned)(N * nchunk)), dim3(RG_THREADS), 0, stream, w, K,
                           nchunk, rotated, codebook, srel, s_channel, u, qpacked);
    else
        hipLaunchKernelGGL(requant_kernel<false>, dim3((unsigned)(N * nchunk)), dim3((unsigned)rg_threads(K)), 0, stream, w, K,
                           nchunk, rotated, codebook, srel, s_channel, u, qpacked);
    return hipGetLastError();
}

hipError_t launch_fake_quant(const float* w_rot, int64_t N, int K, const float* codebook, const uint8_t* srel,
                             const float* s_channel, float* out, hipStream_t stream) {
    (void)hipGetLastError();
    const int64_t groups = N * (K >> 4);
    hipLaunchKernelGGL(fake_quant_kernel, dim3((unsigned)((groups + RG_THREADS - 1) / RG_THREADS)), dim3(RG_THREADS),
                       0, stream, w_rot, groups, K, codebook, srel, s_channel, out);
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* qpacked, const uint8_t* srel, const float* codebook,
                             const float* s_channel, int64_t N, int K, int rotate_back, float* out,
                             hipStream_t stream) {
    (void)hipGetLastError();
    const int nchunk = (K + RG_CHUNK - 1) / RG_CHUNK;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)(N * nchunk)), dim3(RG_THREADS), 0, stream, qpacked, srel,
                       codebook, s_channel, K, nchunk, rotate_back, out);
    return hipGetLastError();
}

}  // namespace w4a8
