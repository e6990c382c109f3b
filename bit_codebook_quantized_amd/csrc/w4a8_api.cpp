// C ABI entry points of libw4a8 (declared in include/w4a8.h).
//
// Every entry point validates its arguments on the host first -- without any HIP
// call -- so a rejected call enqueues and writes nothing.  Then it launches on the
// caller's stream and reports a launch failure as W4A8_ERR_HIP.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4a8.h"

namespace w4a8 {
hipError_t launch_rotate_quant(const uint16_t* x, int64_t M, int K, int qmax, int8_t* xq, float* xs,
                               hipStream_t stream);
hipError_t launch_decode(const uint8_t* qp, const uint8_t* srel, const float* codebook, int64_t N, int K,
                         int8_t* w8, hipStream_t stream);
hipError_t launch_gemv(const int8_t* xq, const float* xs, int M, const uint8_t* qp, const uint8_t* srel,
                       const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                       void* out, hipStream_t stream);
hipError_t launch_gemm(const int8_t* xq, const float* xs, int M, const uint8_t* qp, const uint8_t* srel,
                       const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                       void* out, hipStream_t stream);
hipError_t launch_gemv_grouped(const w4a8_gemv_layer* layers, int count, int M, int out_type, hipStream_t stream);
hipError_t launch_gemv_act(const uint16_t* x, int M, int qmax, const uint8_t* qp, const uint8_t* srel,
                           const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                           void* out, int8_t* xq_out, float* xs_out, hipStream_t stream);
int gemv_act_max_k(int M);
hipError_t launch_requantize(const float* w, int64_t N, int K, int rotated, const float* codebook,
                             const uint8_t* srel, const float* s_channel, const float* u, uint8_t* qpacked,
                             hipStream_t stream);
hipError_t launch_fake_quant(const float* w_rot, int64_t N, int K, const float* codebook, const uint8_t* srel,
                             const float* s_channel, float* out, hipStream_t stream);
hipError_t launch_grad_input(const uint16_t* grad, int M, int N, int K, const uint8_t* qp, const uint8_t* srel,
                             const float* codebook, const float* s_channel, uint16_t* out, hipStream_t stream);
hipError_t launch_lora_merge(const uint8_t* qpacked, const uint8_t* srel, const float* codebook,
                             const float* s_channel, int64_t N, int K, const float* lora_a, const float* lora_b,
                             int rank, float scale, float* out, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* qpacked, const uint8_t* srel, const float* codebook,
                             const float* s_channel, int64_t N, int K, int rotate_back, float* out,
                             hipStream_t stream);
hipError_t launch_empty(int blocks, int threads, hipStream_t stream);
hipError_t launch_quantize(const float* w, int64_t N, int K, int rotated, const float* codebook, uint8_t* qpacked,
                           uint8_t* srel, float* s_channel, hipStream_t stream);
}  // namespace w4a8

namespace {

// Largest M and N accepted: keeps row indices and tile counts in 32-bit range.
constexpr int64_t MAX_ROWS = int64_t(1) << 30;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_k(int64_t K) {
    if (K < 0) return W4A8_ERR_INVALID_ARG;
    if (K < W4A8_ROT_BLOCK || K % W4A8_ROT_BLOCK != 0 || K > W4A8_MAX_K) return W4A8_ERR_SHAPE;
    return W4A8_OK;
}

int check_n(int64_t N) {
    if (N < 0) return W4A8_ERR_INVALID_ARG;
    if (N < 1 || N > MAX_ROWS) return W4A8_ERR_SHAPE;
    return W4A8_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP; }

// Shared checks of w4a8_gemm / w4a8_gemv.
int check_linear(const int8_t* xq, const float* xs, int64_t M, const uint8_t* qpacked, const uint8_t* srel,
                 const float* codebook, const float* s_channel, const float* bias, int64_t N, int64_t K,
                 int32_t group, int32_t out_type, const void* out) {
    if (M < 0) return W4A8_ERR_INVALID_ARG;
    if (M > MAX_ROWS) return W4A8_ERR_SHAPE;
    int st = check_n(N);
    if (st) return st;
    if ((st = check_k(K))) return st;
    if (out_type < W4A8_OUT_BF16 || out_type > W4A8_OUT_SWIGLU_BF16) return W4A8_ERR_INVALID_ARG;
    if (out_type == W4A8_OUT_SWIGLU_BF16 && N % 2 != 0) return W4A8_ERR_SHAPE;
    if (group != W4A8_GROUP) return W4A8_ERR_UNSUPPORTED;
    if (!qpacked || !srel || !codebook || !s_channel) return W4A8_ERR_INVALID_ARG;
    if (M > 0 && (!xq || !xs || !out)) return W4A8_ERR_INVALID_ARG;
    if (!aligned(qpacked, 16) || !aligned(srel, 16) || !aligned(codebook, 4) || !aligned(s_channel, 4) ||
        !aligned(bias, 4))
        return W4A8_ERR_ALIGN;
    if (M > 0 && (!aligned(xq, 16) || !aligned(xs, 4) || !aligned(out, 16))) return W4A8_ERR_ALIGN;
    return W4A8_OK;
}

}  // namespace

extern "C" {

int rotate_quant_act(const void* x, int64_t M, int64_t K, int32_t rot_block, int32_t qmax, int8_t* xq, float* xs,
                     void* stream) {
    if (M < 0) return W4A8_ERR_INVALID_ARG;
    if (M > MAX_ROWS) return W4A8_ERR_SHAPE;
    int st = check_k(K);
    if (st) return st;
    if (rot_block != W4A8_ROT_BLOCK || qmax < 1 || qmax > 127) return W4A8_ERR_UNSUPPORTED;
    if (M == 0) return W4A8_OK;
    if (!x || !xq || !xs) return W4A8_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xs, 4)) return W4A8_ERR_ALIGN;
    return launched(w4a8::launch_rotate_quant(static_cast<const uint16_t*>(x), M, (int)K, qmax, xq, xs,
                                              static_cast<hipStream_t>(stream)));
}

int decode_w4_to_int8(const uint8_t* qpacked, const uint8_t* srel, const float* codebook, int64_t N, int64_t K,
                      int32_t group, int8_t* w8, void* stream) {
    int st = check_n(N);
    if (st) return st;
    if ((st = check_k(K))) return st;
    if (group != W4A8_GROUP) return W4A8_ERR_UNSUPPORTED;
    if (!qpacked || !srel || !codebook || !w8) return W4A8_ERR_INVALID_ARG;
    if (!aligned(qpacked, 16) || !aligned(srel, 16) || !aligned(codebook, 4) || !aligned(w8, 16))
        return W4A8_ERR_ALIGN;
    return launched(w4a8::launch_decode(qpacked, srel, codebook, N, (int)K, w8, static_cast<hipStream_t>(stream)));
}

int w4a8_gemm(const int8_t* xq, const float* xs, int64_t M, const uint8_t* qpacked, const uint8_t* srel,
              const float* codebook, const float* s_channel, const float* bias, int64_t N, int64_t K, int32_t group,
              int32_t out_type, void* out, void* stream) {
    int st = check_linear(xq, xs, M, qpacked, srel, codebook, s_channel, bias, N, K, group, out_type, out);
    if (st) return st;
    if (((M + 255) / 256) * ((N + 127) / 128) > INT32_MAX) return W4A8_ERR_SHAPE;   // output tile count
    if (M == 0) return W4A8_OK;
    return launched(w4a8::launch_gemm(xq, xs, (int)M, qpacked, srel, codebook, s_channel, bias, (int)N, (int)K,
                                      out_type, out, static_cast<hipStream_t>(stream)));
}

int w4a8_gemv(const int8_t* xq, const float* xs, int64_t M, const uint8_t* qpacked, const uint8_t* srel,
              const float* codebook, const float* s_channel, const float* bias, int64_t N, int64_t K, int32_t group,
              int32_t out_type, void* out, void* stream) {
    int st = check_linear(xq, xs, M, qpacked, srel, codebook, s_channel, bias, N, K, group, out_type, out);
    if (st) return st;
    if (M > W4A8_GEMV_MAX_M) return W4A8_ERR_UNSUPPORTED;
    if (M == 0) return W4A8_OK;
    return launched(w4a8::launch_gemv(xq, xs, (int)M, qpacked, srel, codebook, s_channel, bias, (int)N, (int)K,
                                      out_type, out, static_cast<hipStream_t>(stream)));
}

int w4a8_gemv_act(const void* x, int64_t M, int32_t rot_block, int32_t qmax, const uint8_t* qpacked,
                  const uint8_t* srel, const float* codebook, const float* s_channel, const float* bias, int64_t N,
                  int64_t K, int32_t group, int32_t out_type, void* out, int8_t* xq_out, float* xs_out,
                  void* stream) {
    if (M < 0) return W4A8_ERR_INVALID_ARG;
    int st = check_n(N);
    if (st) return st;
    if ((st = check_k(K))) return st;
    if (out_type < W4A8_OUT_BF16 || out_type > W4A8_OUT_SWIGLU_BF16) return W4A8_ERR_INVALID_ARG;
    if (out_type == W4A8_OUT_SWIGLU_BF16 && N % 2 != 0) return W4A8_ERR_SHAPE;
    if (group != W4A8_GROUP || rot_block != W4A8_ROT_BLOCK || qmax < 1 || qmax > 127) return W4A8_ERR_UNSUPPORTED;
    if (M > W4A8_GEMV_MAX_M) return W4A8_ERR_UNSUPPORTED;
    if (!qpacked || !srel || !codebook || !s_channel) return W4A8_ERR_INVALID_ARG;
    if ((xq_out == nullptr) != (xs_out == nullptr)) return W4A8_ERR_INVALID_ARG;
    if (M > 0 && (!x || !out)) return W4A8_ERR_INVALID_ARG;
    if (!aligned(qpacked, 16) || !aligned(srel, 16) || !aligned(codebook, 4) || !aligned(s_channel, 4) ||
        !aligned(bias, 4))
        return W4A8_ERR_ALIGN;
    if (M > 0 && (!aligned(x, 16) || !aligned(out, 16) || !aligned(xq_out, 16) || !aligned(xs_out, 4)))
        return W4A8_ERR_ALIGN;
    if (M == 0) return W4A8_OK;
    if (K > w4a8::gemv_act_max_k((int)M)) return W4A8_ERR_UNSUPPORTED;
    return launched(w4a8::launch_gemv_act(static_cast<const uint16_t*>(x), (int)M, qmax, qpacked, srel, codebook,
                                          s_channel, bias, (int)N, (int)K, out_type, out, xq_out, xs_out,
                                          static_cast<hipStream_t>(stream)));
}

int64_t w4a8_gemv_act_max_k(int64_t M) { return M >= 1 && M <= W4A8_GEMV_MAX_M ? w4a8::gemv_act_max_k((int)M) : 0; }

int w4a8_gemv_grouped(const w4a8_gemv_layer* layers, int32_t count, int64_t M, int32_t group, int32_t out_type,
                      void* stream) {
    if (count < 0 || M < 0) return W4A8_ERR_INVALID_ARG;
    if (M > W4A8_GEMV_MAX_M) return W4A8_ERR_UNSUPPORTED;
    if (count > 0 && !layers) return W4A8_ERR_INVALID_ARG;
    int64_t rows = 0;
    for (int32_t i = 0; i < count; ++i) {
        const w4a8_gemv_layer& L = layers[i];
        const int st = check_linear(L.xq, L.xs, M, L.qpacked, L.srel, L.codebook, L.s_channel, L.bias, L.N, L.K,
                                    group, out_type, L.out);
        if (st) return st;
        rows += L.N;
        if (rows > MAX_ROWS) return W4A8_ERR_SHAPE;
    }
    if (count == 0 || M == 0) return W4A8_OK;
    return launched(w4a8::launch_gemv_grouped(layers, count, (int)M, out_type, static_cast<hipStream_t>(stream)));
}

int quantize_w4(const float* w, int64_t N, int64_t K, int32_t rot_block, int32_t group, int32_t rotated,
                const float* codebook, uint8_t* qpacked, uint8_t* srel, float* s_channel, void* stream) {
    int st = check_n(N);
    if (st) return st;
    if ((st = check_k(K))) return st;
    if (rot_block != W4A8_ROT_BLOCK || group != W4A8_GROUP) return W4A8_ERR_UNSUPPORTED;
    if (!w || !codebook || !qpacked || !srel || !s_channel) return W4A8_ERR_INVALID_ARG;
    if (!aligned(w, 16) || !aligned(codebook, 4) || !aligned(qpacked, 16) || !aligned(srel, 16) ||
        !aligned(s_channel, 4))
        return W4A8_ERR_ALIGN;
    return launched(w4a8::launch_quantize(w, N, (int)K, rotated, codebook, qpacked, srel, s_channel,
                                          static_cast<hipStream_t>(stream)));
}

// Blocks of the row-chunk kernels (one per 4096 columns of a row) must fit a grid.
int check_row_chunks(int64_t N, int64_t K) {
    return N * ((K + 4095) / 4096) > INT32_MAX ? W4A8_ERR_SHAPE : W4A8_OK;
}

int requantize_codes_w4(const float* w, int64_t N, int64_t K, int32_t rot_block, int32_t group, int32_t rotated,
                        const float* codebook, const uint8_t* srel, const float* s_channel, const float* u,
                        uint8_t* qpacked, void* stream) {
    int st = check_n(N);
    if (st) return st;
    if ((st = check_k(K))) return st;
    if ((st = check_row_chunks(N, K))) return st;
    if (rot_block != W4A8_ROT_BLOCK || group != W4A8_GROUP) return W4A8_ERR_UNSUPPORTED;
    if (rotated != 0 && rotated != 1) return W4A8_ERR_INVALID_ARG;
    if (!w || !codebook || !srel || !s_channel || !qpacked) return W4A8_ERR_INVALID_ARG;
    if (!aligned(w, 16) || !aligned(codebook, 4) || !aligned(srel, 16) || !aligned(s_channel, 4) ||
        !aligned(u, 16) || !aligned(qpacked, 16))
        return W4A8_ERR_ALIGN;
    return launched(w4a8::launch_requantize(w, N, (int)K, rotated, codebook, srel, s_channel, u, qpacked,
                                            static_cast<hipStream_t>(stream)));
}

int fake_quant_w4(const float* w_rot, int64_t N, int64_t K, int32_t group, const float* codebook,
                  const uint8_t* srel, const float* s_channel, float* out, void* stream) {
    int st = check_n(N);
    if (st) return st;
    if ((st = check_k(K))) return st;
    if ((st = check_row_chunks(N, K))) return st;
    if (group != W4A8_GROUP) return W4A8_ERR_UNSUPPORTED;
    if (!w_rot || !codebook || !srel || !s_channel || !out) return W4A8_ERR_INVALID_ARG;
    if (!aligned(w_rot, 16) || !aligned(codebook, 4) || !aligned(srel, 16) || !aligned(s_channel, 4) ||
        !aligned(out, 16))
        return W4A8_ERR_ALIGN;
    return launched(w4a8::launch_fake_quant(w_rot, N, (int)K, codebook, srel, s_channel, out,
                                            static_cast<hipStream_t>(stream)));
}

int dequantize_w4(const uint8_t* qpacked, const uint8_t* srel, const float* codebook, const float* s_channel,
                  int64_t N, int64_t K, int32_t rot_block, int32_t group, int32_t rotate_back, float* out,
                  void* stream) {
    int st = check_n(N);
    if (st) return st;
    if ((st = check_k(K))) return st;
    if ((st = check_row_chunks(N, K))) return st;
    if (rot_block != W4A8_ROT_BLOCK || group != W4A8_GROUP) return W4A8_ERR_UNSUPPORTED;
    if (rotate_back != 0 && rotate_back != 1) return W4A8_ERR_INVALID_ARG;
    if (!qpacked || !srel || !codebook || !s_channel || !out) return W4A8_ERR_INVALID_ARG;
    if (!aligned(qpacked, 16) || !aligned(srel, 16) || !aligned(codebook, 4) || !aligned(s_channel, 4) ||
        !aligned(out, 16))
        return W4A8_ERR_ALIGN;
    return launched(w4a8::launch_dequantize(qpacked, srel, codebook, s_channel, N, (int)K, rotate_back, out,
                                            static_cast<hipStream_t>(stream)));
}

int w4a8_grad_input(const void* grad, int64_t M, const uint8_t* qpacked, const uint8_t* srel,
                    const float* codebook, const float* s_channel, int64_t N, int64_t K, int32_t group, void* out,
                    void* stream) {
    if (M < 0) return W4A8_ERR_INVALID_ARG;
    if (M > MAX_ROWS) return W4A8_ERR_SHAPE;
    int st = check_n(N);
    if (st) return st;
    if ((st = check_k(K))) return st;
    if (N % 8 != 0) return W4A8_ERR_SHAPE;
    if (((M + 127) / 128) * (K / 128) > INT32_MAX) return W4A8_ERR_SHAPE;   // output tile count
    if (group != W4A8_GROUP) return W4A8_ERR_UNSUPPORTED;
    if (!qpacked || !srel || !codebook || !s_channel) return W4A8_ERR_INVALID_ARG;
    if (M > 0 && (!grad || !out)) return W4A8_ERR_INVALID_ARG;
    if (!aligned(qpacked, 16) || !aligned(srel, 16) || !aligned(codebook, 4) || !aligned(s_channel, 4))
        return W4A8_ERR_ALIGN;
    if (M > 0 && (!aligned(grad, 16) || !aligned(out, 16))) return W4A8_ERR_ALIGN;
    if (M == 0) return W4A8_OK;
    return launched(w4a8::launch_grad_input(static_cast<const uint16_t*>(grad), (int)M, (int)N, (int)K, qpacked,
                                            srel, codebook, s_channel, static_cast<uint16_t*>(out),
                                            static_cast<hipStream_t>(stream)));
}

int lora_merge_w4(const uint8_t* qpacked, const uint8_t* srel, const float* codebook, const float* s_channel,
                  int64_t N, int64_t K, int32_t rot_block, int32_t group, const float* lora_a, const float* lora_b,
                  int32_t rank, float scale, float* out, void* stream) {
    int st = check_n(N);
    if (st) return st;
    if ((st = check_k(K))) return st;
    if ((st = check_row_chunks(N, K))) return st;
    if (rot_block != W4A8_ROT_BLOCK || group != W4A8_GROUP) return W4A8_ERR_UNSUPPORTED;
    if (rank < 0) return W4A8_ERR_INVALID_ARG;
    if (rank > W4A8_MAX_LORA_RANK) return W4A8_ERR_UNSUPPORTED;
    if (!qpacked || !srel || !codebook || !s_channel || !out) return W4A8_ERR_INVALID_ARG;
    if (rank > 0 && (!lora_a || !lora_b)) return W4A8_ERR_INVALID_ARG;
    if (!aligned(qpacked, 16) || !aligned(srel, 16) || !aligned(codebook, 4) || !aligned(s_channel, 4) ||
        !aligned(out, 16) || !aligned(lora_a, 16) || !aligned(lora_b, 4))
        return W4A8_ERR_ALIGN;
    return launched(w4a8::launch_lora_merge(qpacked, srel, codebook, s_channel, N, (int)K, lora_a, lora_b, rank,
                                            scale, out, static_cast<hipStream_t>(stream)));
}

const char* w4a8_status_string(int status) {
    switch (status) {
        case W4A8_OK: return "W4A8_OK";
        case W4A8_ERR_INVALID_ARG: return "W4A8_ERR_INVALID_ARG";
        case W4A8_ERR_SHAPE: return "W4A8_ERR_SHAPE";
        case W4A8_ERR_ALIGN: return "W4A8_ERR_ALIGN";
        case W4A8_ERR_UNSUPPORTED: return "W4A8_ERR_UNSUPPORTED";
        case W4A8_ERR_HIP: return "W4A8_ERR_HIP";
        default: return "W4A8_ERR_UNKNOWN";
    }
}

int w4a8_empty_launch(int32_t blocks, int32_t threads, void* stream) {
    if (blocks < 1 || blocks > (1 << 20) || threads < 64 || threads > 1024 || threads % 64 != 0)
        return W4A8_ERR_INVALID_ARG;
    return launched(w4a8::launch_empty(blocks, threads, static_cast<hipStream_t>(stream)));
}

int w4a8_abi_version(void) { return 9; }

}  // extern "C"
