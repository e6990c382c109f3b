// w4a8_grad_input: the straight-through backward of the W4A8 layer (ai-toolkit
// convrot_w4a8_quant.py, _w4a8_linear_ste_backward): grad_x[m, k] = sum_n grad[m, n] *
// w[n, k] with w = bf16(bf16(w8[n, k]) * bf16(s_channel[n])), the decoded grid times the
// channel scale in bf16, fp32 accumulation, bf16 output (round to nearest even).  The
// gradient is with respect to the layer's rotated input, as on the page.
//
// A bf16 matrix-core product with the weight decoded on chip (no weight copy in memory):
//   - block tile: 128 output columns (k) x 256 grad rows (m); the contraction (n, the
//     layer's output channels) advances 64 per step; 512 threads = 8 waves, two per SIMD;
//     wave (wk, wm) owns 64 k x 64 m as 4 x 4 tiles of v_mfma_f32_16x16x32_bf16;
//   - operands are swapped (D^T = W^T * grad^T) so each lane's accumulator holds 4
//     consecutive k of one row m: the epilogue stores 8 contiguous bytes;
//   - both operands of a step sit in LDS, n contiguous in 144-byte rows, so a lane's
//     matrix-core operand is one 16-byte read: the grad tile (256 x 64) arrives by
//     full-line loads (8 lanes per 128-byte row), the weight tile (64 n x 128 k) is
//     decoded from one coalesced 8-byte code load per thread (16 codes of one row);
//     partner lanes (rows 2p, 2p + 1) swap a code word, scale byte and channel scale so
//     each converts a pair of rows x 8 columns to bf16 (v_cvt_pk_bf16_f32) and writes it
//     transposed, 16-byte chunks XOR-swizzled by k / 16 (conflict-free writes and reads);
//   - one barrier per step: step s + 2's loads are issued first, and step s + 1's operands
//     (loaded a step earlier) are decoded into the other LDS buffers beside step s's
//     matrix-core work;
//   - tiles are dealt to the 8 XCDs in contiguous ranges of ids, and ids run over bands of
//     2 m-tiles, so the blocks of an XCD share 2 grad panels and half the weight in its L2;
//   - n past N is zero in both operands; rows past M are read clamped, not stored.
#include <type_traits>

#include "w4a8_device.hpp"

namespace w4a8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int GI_THREADS = 512;
constexpr int GI_BK = 128;          // output columns per block
constexpr int GI_BM = 256;          // grad rows per block
constexpr int GI_BN = 64;           // contraction per step
constexpr int GI_PITCH = GI_BN + 8; // bf16 per LDS row (144 bytes: 8 chunks of 16 + pad)
constexpr int GI_WTILE = GI_BK * GI_PITCH;   // bf16 per weight buffer
constexpr int GI_GTILE = GI_BM * GI_PITCH;   // bf16 per grad buffer

struct Stage {
    uint4 g[4];      // 4 x 16 bytes of the grad tile
    uint2 q;         // 16 codes of one weight row
    uint32_t s;      // its scale byte
    float sc;        // its channel scale
};

__global__ __launch_bounds__(GI_THREADS) void grad_input_kernel(const uint16_t* __restrict__ grad, int M, int N,
                                                                 int K, const uint8_t* __restrict__ qp,
                                                                 const uint8_t* __restrict__ srel,
                                                                 const float* __restrict__ codebook,
                                                                 const float* __restrict__ s_channel,
                                                                 uint16_t* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) uint8_t gi_smem[];
    __bf16* wt = reinterpret_cast<__bf16*>(gi_smem);                       // [2][GI_WTILE]
    __bf16* gt = wt + 2 * GI_WTILE;                                          // [2][GI_GTILE]
    uint32_t* lut = reinterpret_cast<uint32_t*>(gt + 2 * GI_GTILE);         // [1024]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave & 1, wm = wave >> 1;
    const int ktiles = K / GI_BK, tiles = (int)gridDim.x;
    // block b runs on XCD b % 8; XCD x takes the contiguous tile range x * tiles / 8 ..
    const int b = blockIdx.x;
    const int t = (tiles % 8 == 0) ? (b % 8) * (tiles / 8) + b / 8 : b;
    // ids run over bands of 2 m-tiles (m fastest within a band): an XCD's 32 tiles at
    // M = 2048, K = 4096 are 2 m-tiles x 16 k-tiles, so it reads 2 grad panels and half of
    // the weight instead of 1 panel and all of it
    const int mtiles = tiles / ktiles, band = t / (2 * ktiles), band_m = min(mtiles - 2 * band, 2);
    const int in_band = t - band * 2 * ktiles;
    const int k0 = (in_band / band_m) * GI_BK, m0 = (2 * band + in_band % band_m) * GI_BM;
    const int KH = K >> 1, G = K >> 4;
    const int nsteps = (N + GI_BN - 1) / GI_BN;
    const int r16 = lane & 15, c4 = lane >> 4;    // fragment row and 8-element chunk

    // code assignment: weight row crow = tid / 8 of the step, group cg = tid % 8 (16 columns);
    // rows 2p (h = 0) and 2p + 1 (h = 1) sit 8 lanes apart
    const int crow = tid >> 3, cg = tid & 7, h = crow & 1, p = crow >> 1;

    auto load = [&](Stage& st, int step) __attribute__((always_inline)) {
        const int sc = min(step, nsteps - 1);   // past the end: a harmless reload
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + GI_THREADS * i, gr = idx >> 3, ch = idx & 7;
            const int m = min(m0 + gr, M - 1);
            const int n = min(sc * GI_BN + 8 * ch, N - 8);
            st.g[i] = *reinterpret_cast<const uint4*>(grad + (int64_t)m * N + n);
        }
        const int n = min(sc * GI_BN + crow, N - 1);
        st.q = *reinterpret_cast<const uint2*>(qp + (int64_t)n * KH + ((k0 + 16 * cg) >> 1));
        st.s = srel[(int64_t)n * G + ((k0 + 16 * cg) >> 4)];
        st.sc = s_channel[n];
    };
    // write step `step`'s operands into buffer `buf`; FULL: the whole step lies below N
    // (every step but a ragged last one), so nothing is zeroed
    auto store_as = [&](auto full, const Stage& st, int step, int buf) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
        const int n0 = step * GI_BN;
        __bf16* gb = gt + buf * GI_GTILE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + GI_THREADS * i, gr = idx >> 3, ch = idx & 7;
            const uint4 v = FULL || n0 + 8 * ch < N ? st.g[i] : uint4{0u, 0u, 0u, 0u};   // N % 8 == 0
            *reinterpret_cast<uint4*>(gb + gr * GI_PITCH + 8 * ch) = v;
        }
        // the partner row's code word for this lane's 8 columns, its scale byte and scale:
        // lane l's partner is l ^ 8, in the same 16-lane row (a DPP rotate by 8, no LDS)
        const uint32_t mine = h ? st.q.y : st.q.x, give = h ? st.q.x : st.q.y;
        const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0x128, 0xF, 0xF, false);
        const uint32_t os = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)st.s, 0x128, 0xF, 0xF, false);
        const float osc = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(st.sc), 0x128, 0xF, 0xF, false));
        const uint32_t qw[2] = {h ? other : mine, h ? mine : other};     // rows 2p, 2p + 1
        const uint32_t sw[2] = {h ? os : st.s, h ? st.s : os};
        const float scw[2] = {h ? osc : st.sc, h ? st.sc : osc};
        float v[2][8];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 tr = reinterpret_cast<const uint4*>(lut)[sw[i]];
            const uint2 d = decode_split(qw[i], tr, 0x03020100u);   // .x even, .y odd columns
            const float sb = (float)(__bf16)scw[i];            // s_channel rounded to bf16
            const bool ok = FULL || n0 + 2 * p + i < N;        // rows past N: zero
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float w8 = (float)(int8_t)(uint8_t)(((j & 1) ? d.y : d.x) >> (8 * (j >> 1)));
                v[i][j] = ok ? __fmul_rn(w8, sb) : 0.0f;          // exact: 8 x 8 significant bits
            }
        }
        // columns 16 * cg + 8 * h + j; the pair (2p, 2p + 1) lies in 16-byte chunk p / 4,
        // swizzled by the column's 16-block (= cg)
        __bf16* wb = wt + buf * GI_WTILE + 8 * ((p >> 2) ^ cg) + 2 * (p & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bf16x2 pr = __builtin_convertvector((f32x2){v[0][j], v[1][j]}, bf16x2);
            *reinterpret_cast<bf16x2*>(wb + (16 * cg + 8 * h + j) * GI_PITCH) = pr;
        }
    };
    auto store = [&](const Stage& st, int step, int buf) __attribute__((always_inline)) {
        if (step * GI_BN + GI_BN <= N)   // block-uniform
            store_as(std::true_type{}, st, step, buf);
        else
            store_as(std::false_type{}, st, step, buf);
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = (f32x4){0.f, 0.f, 0.f, 0.f};

    auto mma = [&](int buf) __attribute__((always_inline)) {
        const __bf16* wb = wt + buf * GI_WTILE;
        const __bf16* gb = gt + buf * GI_GTILE;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            bf16x8 bf[4];
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
                bf[ms] = *reinterpret_cast<const bf16x8*>(gb + (64 * wm + 16 * ms + r16) * GI_PITCH + 32 * hh + 8 * c4);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int krow = 64 * wk + 16 * ks + r16;                // (krow >> 4) = 4 wk + ks
                const int chunk = (4 * hh + c4) ^ ((4 * wk + ks) & 7);
                const bf16x8 af = *reinterpret_cast<const bf16x8*>(wb + krow * GI_PITCH + 8 * chunk);
#pragma unroll
                for (int ms = 0; ms < 4; ++ms)
                    acc[ks][ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[ms], acc[ks][ms], 0, 0, 0);
            }
        }
    };

    // prologue: level table, step 0's operands in buffer 0, step 1's loads in flight
    Stage sa, sb;
    load(sa, 0);
    float cbv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) cbv[c] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(codebook[c])));
    build_level_table_regs(lut, cbv, tid, GI_THREADS);
    __syncthreads();
    store(sa, 0, 0);
    load(sa, 1);
    __syncthreads();

    // Step s: the loads of step s + 2 are issued first; then step s + 1's operands, loaded
    // a whole step earlier, are decoded and written into the other buffer while step s's
    // matrix-core work reads this one, so the two interleave; one barrier ends the step.
    // Two named stages alternate (no register copies).  Past the end the loads re-read the
    // last step and the writes are zeros (n >= N) that nobody reads.
    auto step = [&](int s, Stage& cur, Stage& nxt) __attribute__((always_inline)) {
        load(nxt, s + 2);
        __builtin_amdgcn_sched_barrier(0);   // the loads stay ahead of this step's work
        store(cur, s + 1, (s + 1) & 1);
        mma(s & 1);
        __syncthreads();
    };
    int s = 0;
    for (; s + 2 <= nsteps; s += 2) {
        step(s, sa, sb);
        step(s + 1, sb, sa);
    }
    if (s < nsteps) step(s, sa, sb);

    // epilogue: lane holds D[k = 4 * c4 + r][m = r16] of each 16 x 16 tile
    if (m0 + GI_BM <= M) {
        // whole tile: each wave passes its 64 x 64 outputs through LDS (the operand buffers,
        // free after the last barrier; 144-byte rows) and stores each row's 128 bytes with 8
        // lanes, whole lines, as non-temporal stores (the output is not read again here)
        constexpr int OP = 144;
        uint8_t* ob = gi_smem + wave * (64 * OP);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const f32x4 a = acc[ks][ms];
                const bf16x2 lo = __builtin_convertvector((f32x2){a[0], a[1]}, bf16x2);
                const bf16x2 hi = __builtin_convertvector((f32x2){a[2], a[3]}, bf16x2);
                *reinterpret_cast<uint2*>(ob + (16 * ms + r16) * OP + 2 * (16 * ks + 4 * c4)) =
                    uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            }
        wave_lds_sync();   // the wave's own rows: ordered within the wave
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = (lane >> 3) + 8 * i, c = lane & 7;
            const uint4 v = *reinterpret_cast<const uint4*>(ob + row * OP + 16 * c);
            const int64_t m = m0 + 64 * wm + row;
            __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w},
                                        reinterpret_cast<u32x4*>(out + m * K + k0 + 64 * wk + 8 * c));
        }
        return;
    }
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
    const size_t lds = (size_t)(2 * GI_WTILE + 2 * GI_GTILE) * 2 + 4096;   // 114,688 bytes
    hipLaunchKernelGGL(grad_input_kernel, dim3((unsigned)blocks), dim3(GI_THREADS), lds, stream, grad, M, N, K, qp,
                       srel, codebook, s_channel, out);
    return hipGetLastError();
}

}  // namespace w4a8
