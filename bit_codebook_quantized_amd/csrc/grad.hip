// w4a8_grad_input: the straight-through backward of the W4A8 layer (ai-toolkit
// convrot_w4a8_quant.py, _w4a8_linear_ste_backward): grad_x[m, k] = sum_n grad[m, n] *
// w[n, k] with w = bf16(bf16(w8[n, k]) * bf16(s_channel[n])), the decoded grid times the
// channel scale in bf16, fp32 accumulation, bf16 output (round to nearest even).  The
// gradient is with respect to the layer's rotated input, as on the page.
//
// A bf16 matrix-core product with the weight decoded on chip (no weight copy in memory):
//   - block tile: 128 output columns (k) x 256 grad rows (m); the contraction (n, the
//     layer's output channels) advances 64 per step; 512 threads = 8 waves, two per SIMD
//     (the register budget is held to that), so one wave's matrix-core work overlaps the
//     other's decode; wave (wk, wm) owns 64 k x 64 m as 4 x 4 tiles of
//     v_mfma_f32_16x16x32_bf16;
//   - operands are swapped (D^T = W^T * grad^T) so each lane's accumulator holds 4
//     consecutive k of one row m: the epilogue stores 8 contiguous bytes;
//   - grad fragments (8 consecutive n of one row per lane) are loaded straight from
//     memory into registers, one step ahead;
//   - the weight tile of a step (64 n x 128 k) is decoded once for all 256 rows -- thread
//     t takes rows 2p, 2p+1 (p = t % 32) and the 8 columns 8 * (t / 32) -- through the LDS
//     level table, scaled, converted to bf16 in pairs of rows (v_cvt_pk_bf16_f32) and
//     written transposed (k-major, n contiguous, 144-byte rows: conflict-free reads and
//     writes) into one of two LDS buffers, so a lane's matrix-core operand is one 16-byte
//     read;
//   - tiles are dealt to the 8 XCDs in contiguous ranges, m-major, so the blocks of an
//     XCD share their grad rows in its L2;
//   - rows past N are zero in both operands; rows past M are read clamped, not stored.
#include <type_traits>

#include "w4a8_device.hpp"

namespace w4a8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int GI_THREADS = 512;
constexpr int GI_BK = 128;          // output columns per block
constexpr int GI_BM = 256;          // grad rows per block
constexpr int GI_BN = 64;           // contraction per step
constexpr int GI_PITCH = GI_BN + 8; // bf16 per row of the transposed weight tile (144 bytes)
constexpr int GI_TILE = GI_BK * GI_PITCH;   // bf16 per buffer

struct GFrag {
    uint4 v[2][4];   // [32-n half][m subtile]
};

struct Codes {
    uint32_t q[2];   // two rows' 8 codes of the thread's columns
    uint32_t s[2];   // their scale bytes
    float sc[2];     // their channel scales
};

__device__ __forceinline__ uint32_t zero_tail(uint32_t w, int i, int valid) {
    // elements 2i (low half) and 2i + 1 (high half) of a fragment; keep those < valid
    const uint32_t lo = 2 * i < valid ? 0x0000FFFFu : 0u, hi = 2 * i + 1 < valid ? 0xFFFF0000u : 0u;
    return w & (lo | hi);
}

__global__ __launch_bounds__(GI_THREADS) void grad_input_kernel(const uint16_t* __restrict__ grad, int M, int N,
                                                                 int K, const uint8_t* __restrict__ qp,
                                                                 const uint8_t* __restrict__ srel,
                                                                 const float* __restrict__ codebook,
                                                                 const float* __restrict__ s_channel,
                                                                 uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) __bf16 wt[2][GI_TILE];
    __shared__ __attribute__((aligned(16))) uint32_t lut[1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave & 1, wm = wave >> 1;
    const int ktiles = K / GI_BK, tiles = (int)gridDim.x;
    // block b runs on XCD b % 8; XCD x takes the contiguous tile range x * tiles / 8 ..
    const int b = blockIdx.x;
    const int t = (tiles % 8 == 0) ? (b % 8) * (tiles / 8) + b / 8 : b;
    const int k0 = (t % ktiles) * GI_BK, m0 = (t / ktiles) * GI_BM;
    const int KH = K >> 1, G = K >> 4;
    const int nsteps = (N + GI_BN - 1) / GI_BN;
    const int r16 = lane & 15, c4 = lane >> 4;    // fragment row and 8-element chunk

    // decode assignment: row pair p, columns kcol .. kcol + 7
    const int p = tid & 31, hg = tid >> 5;
    const int kcol = k0 + 8 * hg;

    auto load_codes = [&](Codes& c, int step) __attribute__((always_inline)) {
        step = min(step, nsteps - 1);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int n = min(step * GI_BN + 2 * p + i, N - 1);
            c.q[i] = *reinterpret_cast<const uint32_t*>(qp + (int64_t)n * KH + (kcol >> 1));
            c.s[i] = srel[(int64_t)n * G + (kcol >> 4)];
            c.sc[i] = s_channel[n];
        }
    };
    auto load_grad = [&](GFrag& g, int step) __attribute__((always_inline)) {
        step = min(step, nsteps - 1);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                const int m = min(m0 + 64 * wm + 16 * ms + r16, M - 1);
                const int n = min(step * GI_BN + 32 * h + 8 * c4, ((N - 1) & ~7));
                g.v[h][ms] = *reinterpret_cast<const uint4*>(grad + (int64_t)m * N + n);
            }
    };
    // decoded, scaled, bf16 pairs of rows written transposed into buffer b
    auto decode = [&](const Codes& c, int step, int buf, auto masked) __attribute__((always_inline)) {
        const int nb = step * GI_BN + 2 * p;
        float v[2][8];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 tr = reinterpret_cast<const uint4*>(lut)[c.s[i]];
            const uint2 d = decode8(c.q[i], tr);
            const float sb = (float)(__bf16)c.sc[i];            // s_channel rounded to bf16
            const bool ok = !decltype(masked)::value || nb + i < N;   // rows past N: zero
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float w8 = (float)(int8_t)(uint8_t)((j < 4 ? d.x : d.y) >> (8 * (j & 3)));
                v[i][j] = ok ? __fmul_rn(w8, sb) : 0.0f;          // exact: 8 x 8 significant bits
            }
        }
        __bf16* dst = wt[buf] + 2 * p;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bf16x2 pr = __builtin_convertvector((f32x2){v[0][j], v[1][j]}, bf16x2);
            *reinterpret_cast<bf16x2*>(dst + (8 * hg + j) * GI_PITCH) = pr;
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

    auto mma = [&](const GFrag& g, int step, int buf, auto masked) __attribute__((always_inline)) {
        const int valid = N - (step * GI_BN);   // n still inside the layer, from this step's start
        constexpr bool tail = decltype(masked)::value;   // only the last steps reach past N
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int vchunk = valid - (32 * h + 8 * c4);     // valid elements of this lane's chunk
            bf16x8 bf[4];
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                uint4 u = g.v[h][ms];
                if (tail) {   // the contraction's tail: zero the elements past N
                    u.x = zero_tail(u.x, 0, vchunk); u.y = zero_tail(u.y, 1, vchunk);
                    u.z = zero_tail(u.z, 2, vchunk); u.w = zero_tail(u.w, 3, vchunk);
                }
                bf[ms] = __builtin_bit_cast(bf16x8, u);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 af = *reinterpret_cast<const bf16x8*>(
                    wt[buf] + (64 * wk + 16 * ks + r16) * GI_PITCH + 32 * h + 8 * c4);
#pragma unroll
                for (int ms = 0; ms < 4; ++ms)
                    acc[ks][ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[ms], acc[ks][ms], 0, 0, 0);
            }
        }
    };

    // prologue: level table, step 0 decoded, step 1's codes and step 0's grad in flight
    Codes ca, cb;
    GFrag ga, gb;
    load_codes(ca, 0);
    load_grad(ga, 0);
    float cbv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) cbv[c] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(codebook[c])));
    build_level_table_regs(lut, cbv, tid, GI_THREADS);
    __syncthreads();
    decode(ca, 0, 0, std::true_type{});
    load_codes(cb, 1);
    __syncthreads();

    // Two steps per trip with no early exit: a conditional second half would let the
    // compiler sink its prefetch into it.  A padding step past the end (odd step count)
    // multiplies zeros: its weight rows decode to zero and its grad fragments are masked.
    // Full steps run unmasked; the last one or two (n past N, or the padding step) run the
    // masked form, a separate copy of the pair.
    // `next_masked`: whether step s + 2 (decoded here for the next pair) may reach past N
    auto pair = [&](int s, auto masked, auto next_masked) __attribute__((always_inline)) {
        load_grad(gb, s + 1);
        __builtin_amdgcn_sched_barrier(0);   // the prefetch stays ahead of the computation
        mma(ga, s, 0, masked);
        decode(cb, s + 1, 1, masked);
        load_codes(ca, s + 2);
        __syncthreads();
        load_grad(ga, s + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma(gb, s + 1, 1, masked);
        decode(ca, s + 2, 0, next_masked);
        load_codes(cb, s + 3);
        __syncthreads();
    };
    const int nfull = N / GI_BN;
    int s = 0;
    for (; s + 4 <= nfull; s += 2) pair(s, std::false_type{}, std::false_type{});
    if (s + 2 <= nfull) {
        pair(s, std::false_type{}, std::true_type{});
        s += 2;
    }
    if (s < nsteps) pair(s, std::true_type{}, std::true_type{});   // at most two steps remain

    // epilogue: lane holds D[k = 4 * c4 + r][m = r16] of each 16 x 16 tile
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
        const int m = m0 + 64 * wm + 16 * ms + r16;
        if (m >= M) continue;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int k = k0 + 64 * wk + 16 * ks + 4 * c4;
            const f32x4 a = acc[ks][ms];
            const bf16x2 lo = __builtin_convertvector((f32x2){a[0], a[1]}, bf16x2);
            const bf16x2 hi = __builtin_convertvector((f32x2){a[2], a[3]}, bf16x2);
            *reinterpret_cast<uint2*>(out + (int64_t)m * K + k) =
                uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
    }
}

}  // namespace

hipError_t launch_grad_input(const uint16_t* grad, int M, int N, int K, const uint8_t* qp, const uint8_t* srel,
                             const float* codebook, const float* s_channel, uint16_t* out, hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    const int64_t blocks = (int64_t)(K / GI_BK) * ((M + GI_BM - 1) / GI_BM);   // one block per tile
    hipLaunchKernelGGL(grad_input_kernel, dim3((unsigned)blocks), dim3(GI_THREADS), 0, stream, grad, M, N, K, qp,
                       srel, codebook, s_channel, out);
    return hipGetLastError();
}

}  // namespace w4a8
