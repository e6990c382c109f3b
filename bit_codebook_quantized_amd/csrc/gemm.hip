// w4a8_gemm: prefill product for any M on the int8 matrix cores of gfx950.
//
// ai-toolkit convrot_w4a8_quant.py, _w4a8_linear_ste_op: the int8 grid of the
// weight (decoded from 4-bit codes, fp8 group scales and the codebook) times the
// int8 activation rows, accumulated exactly in int32, then the epilogue
// fp32(acc) * (xs[m] * ws[n]) [+ bias[n]].  Unlike the page, which writes the
// decoded int8 weight to memory and runs a library int8 GEMM on it, the weight is
// decoded tile by tile into LDS here, so no int8 weight copy ever reaches HBM.
//
// Tiling: one block of 256 threads (4 waves) computes a BM x BN = 256 x 128 output
// tile, stepping K by BK = 64.  Per step every thread loads 4 x 16 B of activation
// rows and 16 B of packed codes plus 2 scale bytes (one row, 32 columns, two
// groups), decodes the codes with byte permutes against the LDS level table and
// stores both tiles into a double-buffered LDS stage (rows padded to 80 B so the
// 16-byte fragment reads of 16 consecutive rows hit distinct banks).  The waves
// form a 2 x 2 grid of 128 x 64 sub-tiles, each 4 x 2 v_mfma_i32_32x32x32_i8
// accumulators (128 int32 registers per lane).  Both MFMA operands are read as
// 16 consecutive k bytes per lane (lane % 32 = row, lane / 32 = which 16-byte
// half of the 32-wide k step), so A and B agree on the k order by construction.
//
// Tiles are mapped to blocks so that each of the 8 XCDs (blocks are dealt to
// XCDs round robin) works on a contiguous range of tile ids, n fastest, which
// keeps one activation row-panel and neighbouring weight panels in its L2.
#include "w4a8_device.hpp"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int GM_THREADS = 256;
constexpr int BM = 256, BN = 128, BK = 64;
constexpr int LDSTRIDE = BK + 16;   // bytes per LDS row
constexpr int DEPTH = 4;            // K-steps of global loads in flight

template <int OUT>
__global__ __launch_bounds__(GM_THREADS, 1) void gemm_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int M, const uint8_t* __restrict__ qp,
    const uint8_t* __restrict__ srel, const float* __restrict__ codebook, const float* __restrict__ ws,
    const float* __restrict__ bias, int N, int K, int out_type, void* __restrict__ out, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint32_t lut[1024];
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * LDSTRIDE];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * LDSTRIDE];
    __shared__ float xs_t[BM], ws_t[BN], bias_t[BN];   // the tile's epilogue scales

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ntiles = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);
    const int tn = pid % tiles_n, tm = pid / tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    build_level_table(lut, codebook, tid, GM_THREADS);
    const uint4* lut4 = reinterpret_cast<const uint4*>(lut);
    // epilogue operands of this tile, staged once (rows/columns past the edge get 0)
    xs_t[tid] = m0 + tid < M ? xs[m0 + tid] : 0.0f;
    if (tid < BN) {
        ws_t[tid] = n0 + tid < N ? ws[n0 + tid] : 0.0f;
        bias_t[tid] = (bias && n0 + tid < N) ? bias[n0 + tid] : 0.0f;
    }

    // global -> register roles
    const int a_row = tid >> 2, a_chk = tid & 3;
    const int b_row = tid >> 1, b_half = tid & 1;
    const int KH = K >> 1, G = K >> 4;
    const bool b_ok = n0 + b_row < N;
    const uint8_t* qp_row = qp + (int64_t)(b_ok ? n0 + b_row : 0) * KH + b_half * 16;
    // the 4 scale bytes of a K-step are one aligned dword; this thread uses 2 of them
    const uint8_t* sr_row = srel + (int64_t)(b_ok ? n0 + b_row : 0) * G;
    const int s_shift = 16 * b_half;
    // Rows past M (and columns past N) load row 0: they only feed accumulators whose
    // outputs are never stored, so no masking is needed.
    const int8_t* a_ptr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int mr = m0 + a_row + 64 * p;
        a_ptr[p] = xq + (int64_t)(mr < M ? mr : 0) * K + a_chk * 16;
    }

    // Register ring of in-flight global loads: slot d holds K-step kt with kt % DEPTH == d.
    // Step kt+1 is written to LDS while step kt is multiplied, and its slot is refilled
    // with step kt+1+DEPTH, so every global load has DEPTH steps of MFMA work to land.
    struct Stage {   // native vector registers only, so the stage lives in VGPRs
        v4u a0, a1, a2, a3;
        v4u b;
        uint32_t s;
    };
    // Loads are unconditional (rows past M or N read row 0, steps past the end re-read
    // the last step) so the count of loads in flight is the same on every path and the
    // compiler can wait for exactly the oldest stage instead of draining all of them.
    auto gload = [&](Stage& st, int kt) __attribute__((always_inline)) {
        const int k0 = kt * BK;
        st.a0 = *reinterpret_cast<const v4u*>(a_ptr[0] + k0);
        st.a1 = *reinterpret_cast<const v4u*>(a_ptr[1] + k0);
        st.a2 = *reinterpret_cast<const v4u*>(a_ptr[2] + k0);
        st.a3 = *reinterpret_cast<const v4u*>(a_ptr[3] + k0);
        st.b = *reinterpret_cast<const v4u*>(qp_row + (k0 >> 1));
        st.s = *reinterpret_cast<const uint32_t*>(sr_row + (k0 >> 4));
    };
    auto lstore = [&](const Stage& st, int buf) __attribute__((always_inline)) {
        int8_t* arow = &As[buf][a_row * LDSTRIDE + a_chk * 16];
        *reinterpret_cast<v4u*>(arow) = st.a0;
        *reinterpret_cast<v4u*>(arow + 64 * LDSTRIDE) = st.a1;
        *reinterpret_cast<v4u*>(arow + 128 * LDSTRIDE) = st.a2;
        *reinterpret_cast<v4u*>(arow + 192 * LDSTRIDE) = st.a3;
        const uint4 t0 = lut4[(st.s >> s_shift) & 0xFFu], t1 = lut4[(st.s >> (s_shift + 8)) & 0xFFu];
        const uint2 d0 = decode8(st.b.x, t0), d1 = decode8(st.b.y, t0);
        const uint2 d2 = decode8(st.b.z, t1), d3 = decode8(st.b.w, t1);
        v4u* dst = reinterpret_cast<v4u*>(&Bs[buf][b_row * LDSTRIDE + b_half * 32]);
        dst[0] = v4u{d0.x, d0.y, d1.x, d1.y};
        dst[1] = v4u{d2.x, d2.y, d3.x, d3.y};
    };

    const int wm = wave >> 1, wn = wave & 1;
    v16i acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int nk = K / BK;   // a multiple of DEPTH because K % 256 == 0
    // The ring is four named stages (no indexed array: an indexed private array could be
    // placed in memory by the compiler, which would serialise the loads).
    Stage r0, r1, r2, r3;
    gload(r0, 0);
    gload(r1, 1);
    gload(r2, 2);
    gload(r3, 3);
    __syncthreads();   // level table ready
    lstore(r0, 0);
    gload(r0, min(DEPTH, nk - 1));
    __syncthreads();

    const int frag_row = lane & 31, frag_k = (lane >> 5) * 16;
    // one K-step: multiply LDS buffer `buf` (step kt), stage step kt+1 from `st` into the
    // other buffer, refill `st` with step kt+1+DEPTH
    auto step = [&](int kt, int buf, Stage& st) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v4i af[4], bf[2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                af[mt] = *reinterpret_cast<const v4i*>(
                    &As[buf][(wm * 128 + mt * 32 + frag_row) * LDSTRIDE + ks * 32 + frag_k]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                bf[nt] = *reinterpret_cast<const v4i*>(
                    &Bs[buf][(wn * 64 + nt * 32 + frag_row) * LDSTRIDE + ks * 32 + frag_k]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
        }
        lstore(st, buf ^ 1);   // past the end: a harmless rewrite of a buffer nobody reads
        gload(st, min(kt + 1 + DEPTH, nk - 1));
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt0 = 0; kt0 < nk; kt0 += DEPTH) {
        step(kt0 + 0, 0, r1);
        step(kt0 + 1, 1, r2);
        step(kt0 + 2, 0, r3);
        step(kt0 + 3, 1, r0);
    }

    // epilogue: accumulator register r of a 32 x 32 tile holds row 8*(r/4) + 4*(lane/32) + r%4,
    // column lane % 32; stores of rows past M / columns past N are skipped
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int nl = wn * 64 + nt * 32 + (lane & 31), n = n0 + nl;
        const float wsn = ws_t[nl], bn = bias_t[nl];
        const bool n_ok = n < N;
        const bool interior = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ml = wm * 128 + mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), m = m0 + ml;
                const int32_t a = acc[mt][nt][r];
                float y = __fmul_rn((float)a, __fmul_rn(xs_t[ml], wsn));
                if (bias) y = __fadd_rn(y, bn);
                if (interior || (n_ok && m < M)) store_out(out, OUT, (int64_t)m * N + n, a, y);
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* xs, int M, const uint8_t* qp, const uint8_t* srel,
                       const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                       void* out, hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t ntiles = (int64_t)tiles_m * tiles_n;
    const dim3 g((unsigned)ntiles), b(GM_THREADS);
    if (out_type == 0)
        hipLaunchKernelGGL(gemm_kernel<0>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out_type,
                           out, tiles_m, tiles_n);
    else if (out_type == 1)
        hipLaunchKernelGGL(gemm_kernel<1>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out_type,
                           out, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL(gemm_kernel<2>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out_type,
                           out, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace w4a8
