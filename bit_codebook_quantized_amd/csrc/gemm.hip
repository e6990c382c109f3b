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
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int GM_THREADS = 256;
constexpr int BM = 256, BN = 128, BK = 64;
constexpr int LDSTRIDE = BK + 16;   // bytes per LDS row

__global__ __launch_bounds__(GM_THREADS, 1) void gemm_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int M, const uint8_t* __restrict__ qp,
    const uint8_t* __restrict__ srel, const float* __restrict__ codebook, const float* __restrict__ ws,
    const float* __restrict__ bias, int N, int K, int out_type, void* __restrict__ out, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint32_t lut[1024];
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * LDSTRIDE];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * LDSTRIDE];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ntiles = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);
    const int tn = pid % tiles_n, tm = pid / tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    build_level_table(lut, codebook, tid, GM_THREADS);
    const uint4* lut4 = reinterpret_cast<const uint4*>(lut);

    // global -> register roles
    const int a_row = tid >> 2, a_chk = tid & 3;
    const int b_row = tid >> 1, b_half = tid & 1;
    const int KH = K >> 1, G = K >> 4;
    const bool b_ok = n0 + b_row < N;
    const uint8_t* qp_row = qp + (int64_t)(b_ok ? n0 + b_row : 0) * KH + b_half * 16;
    const uint8_t* sr_row = srel + (int64_t)(b_ok ? n0 + b_row : 0) * G + b_half * 2;
    const int8_t* a_ptr[4];
    bool a_ok[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int mr = m0 + a_row + 64 * p;
        a_ok[p] = mr < M;
        a_ptr[p] = xq + (int64_t)(a_ok[p] ? mr : 0) * K + a_chk * 16;
    }

    uint4 ra[4], rb;
    uint32_t rs;
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            ra[p] = a_ok[p] ? *reinterpret_cast<const uint4*>(a_ptr[p] + k0) : make_uint4(0, 0, 0, 0);
        rb = b_ok ? *reinterpret_cast<const uint4*>(qp_row + (k0 >> 1)) : make_uint4(0, 0, 0, 0);
        rs = b_ok ? (uint32_t)*reinterpret_cast<const uint16_t*>(sr_row + (k0 >> 4)) : 0u;
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<uint4*>(&As[buf][(a_row + 64 * p) * LDSTRIDE + a_chk * 16]) = ra[p];
        const uint4 t0 = lut4[rs & 0xFFu], t1 = lut4[rs >> 8];
        const uint2 d0 = decode8(rb.x, t0), d1 = decode8(rb.y, t0);
        const uint2 d2 = decode8(rb.z, t1), d3 = decode8(rb.w, t1);
        uint4* dst = reinterpret_cast<uint4*>(&Bs[buf][b_row * LDSTRIDE + b_half * 32]);
        dst[0] = make_uint4(d0.x, d0.y, d1.x, d1.y);
        dst[1] = make_uint4(d2.x, d2.y, d3.x, d3.y);
    };

    const int wm = wave >> 1, wn = wave & 1;
    v16i acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int nk = K / BK;
    gload(0);
    __syncthreads();   // level table ready
    lstore(0);
    __syncthreads();

    const int frag_row = lane & 31, frag_k = (lane >> 5) * 16;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
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
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: accumulator register r of a 32 x 32 tile holds row 8*(r/4) + 4*(lane/32) + r%4,
    // column lane % 32
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int n = n0 + wn * 64 + nt * 32 + (lane & 31);
            if (n >= N) continue;
            const float wsn = ws[n];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 128 + mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M) {
                    const int32_t a = acc[mt][nt][r];
                    const float y = epilogue_f32(a, xs[m], wsn, bias, n);
                    store_out(out, out_type, (int64_t)m * N + n, a, y);
                }
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
    hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)ntiles), dim3(GM_THREADS), 0, stream, xq, xs, M, qp, srel,
                       codebook, ws, bias, N, K, out_type, out, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace w4a8
