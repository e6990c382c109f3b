// w4a8_gemv: decode-path product for M <= 8 token rows, on the vector ALUs.
//
// ai-toolkit convrot_w4a8_quant.py, w4a8_gemv_kernel: the packed codes, the fp8
// group scales and the codebook are read directly, every weight is decoded to its
// int8 grid value in registers and multiply-accumulated in int32 against the int8
// activation rows (exact, so the result equals the matrix-core path bit for bit),
// and the epilogue fp32(acc) * (xs[m] * ws[n]) [+ bias[n]] is fused into the store.
// Weight traffic is 4 bits per code plus one scale byte per 16 codes (4.5 bit per
// weight), which bounds the kernel by HBM bandwidth.
//
// Layout: a block of 256 threads = 4 waves; wave w owns R consecutive output rows
// and its 64 lanes split K in 16-column chunks (one 8-byte load of codes, one scale
// byte).  Per chunk a lane loads the M activation chunks once and reuses them for
// its R rows.  The int32 partial sums stay in registers until the end of K and are
// then summed across the wave once.  v_dot4_i32_i8 does four products per
// instruction; the decode is done with byte permutes against the 16-level table
// row of the group's scale byte (level table in LDS, built once per block).
#include "w4a8_device.hpp"

namespace w4a8 {
namespace {

constexpr int GV_THREADS = 256;

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int MM, int R>
__global__ __launch_bounds__(GV_THREADS) void gemv_kernel(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                          const uint8_t* __restrict__ qp,
                                                          const uint8_t* __restrict__ srel,
                                                          const float* __restrict__ codebook,
                                                          const float* __restrict__ ws,
                                                          const float* __restrict__ bias, int N, int K,
                                                          int out_type, void* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint32_t lut[1024];
    build_level_table(lut, codebook, threadIdx.x, GV_THREADS);
    __syncthreads();
    const uint4* lut4 = reinterpret_cast<const uint4*>(lut);

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * (GV_THREADS / 64) + wave) * R;
    const int KH = K >> 1, G = K >> 4, nchunk = K >> 4;

    const uint8_t* qrow[R];
    const uint8_t* srow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int n = min(n0 + r, N - 1);
        qrow[r] = qp + (int64_t)n * KH;
        srow[r] = srel + (int64_t)n * G;
    }

    int32_t acc[R][MM];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[r][m] = 0;

    for (int j = lane; j < nchunk; j += 64) {
        uint4 a[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) a[m] = *reinterpret_cast<const uint4*>(xq + (int64_t)m * K + j * 16);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint2 p = *reinterpret_cast<const uint2*>(qrow[r] + j * 8);
            const uint4 t = lut4[srow[r][j]];
            const uint2 d0 = decode8(p.x, t), d1 = decode8(p.y, t);
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                int32_t s = acc[r][m];
                s = __builtin_amdgcn_sdot4((int)d0.x, (int)a[m].x, s, false);
                s = __builtin_amdgcn_sdot4((int)d0.y, (int)a[m].y, s, false);
                s = __builtin_amdgcn_sdot4((int)d1.x, (int)a[m].z, s, false);
                s = __builtin_amdgcn_sdot4((int)d1.y, (int)a[m].w, s, false);
                acc[r][m] = s;
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[r][m] = wave_sum(acc[r][m]);

#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int n = n0 + r;
            if (lane == r * MM + m && n < N) {
                const float y = epilogue_f32(acc[r][m], xs[m], ws[n], bias, n);
                store_out(out, out_type, (int64_t)m * N + n, acc[r][m], y);
            }
        }
    }
}

template <int MM>
hipError_t launch_gemv_m(const int8_t* xq, const float* xs, const uint8_t* qp, const uint8_t* srel,
                         const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                         void* out, hipStream_t stream) {
    // rows per wave: enough waves to cover the 256 compute units several times
    const int waves_per_block = GV_THREADS / 64;
    int R = 4;
    if ((N + 3) / 4 < 4 * 256) R = 2;
    if ((N + 1) / 2 < 4 * 256) R = 1;
    const int blocks = (N + waves_per_block * R - 1) / (waves_per_block * R);
    const dim3 g(blocks), b(GV_THREADS);
    if (R == 4)
        hipLaunchKernelGGL((gemv_kernel<MM, 4>), g, b, 0, stream, xq, xs, qp, srel, codebook, ws, bias, N, K,
                           out_type, out);
    else if (R == 2)
        hipLaunchKernelGGL((gemv_kernel<MM, 2>), g, b, 0, stream, xq, xs, qp, srel, codebook, ws, bias, N, K,
                           out_type, out);
    else
        hipLaunchKernelGGL((gemv_kernel<MM, 1>), g, b, 0, stream, xq, xs, qp, srel, codebook, ws, bias, N, K,
                           out_type, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const int8_t* xq, const float* xs, int M, const uint8_t* qp, const uint8_t* srel,
                       const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                       void* out, hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    switch (M) {
        case 1: return launch_gemv_m<1>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 2: return launch_gemv_m<2>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 3: return launch_gemv_m<3>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 4: return launch_gemv_m<4>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 5: return launch_gemv_m<5>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 6: return launch_gemv_m<6>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 7: return launch_gemv_m<7>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 8: return launch_gemv_m<8>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a8
