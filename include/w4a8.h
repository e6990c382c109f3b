/*
 * w4a8.h -- C ABI of the ConvRot W4A8 codebook linear layer on AMD MI355X (gfx950).
 *
 * The layer (ai-toolkit, toolkit/util/convrot_w4a8_quant.py: module docstring and
 * class ConvRotW4A8Quantizer) computes, for bf16 activations x [M, K]:
 *
 *   1. xr    = x rotated block-wise by the normalised regular Hadamard matrix of
 *              size 256 (h3-rs 0.2.0, src/weights.rs: fn hadamard, fn rotate_activation);
 *   2. xq,xs = per-token symmetric int8 quantisation of xr (ai-toolkit:
 *              w4a8_act_quant_kernel);
 *   3. w8    = the int8 grid decoded from packed 4-bit codebook indices and fp8-e4m3
 *              group scales (ai-toolkit: storage contract, unpack_w4a8_eager, W4A8_SAT);
 *   4. acc   = xq * w8^T exactly in int32;
 *   5. y     = fp32(acc) * (xs[m] * s_channel[n]) [+ bias[n]] cast to the output type
 *              (ai-toolkit: w4a8_gemv_kernel epilogue).
 *
 * Storage of one layer with N output channels and K input channels (K % 256 == 0):
 *   qpacked   uint8 [N, K/2]   row-major; byte j of a row holds the code of column 2j in
 *                              bits 0..3 and of column 2j+1 in bits 4..7 (codes 0..15).
 *   srel      uint8 [N, K/16]  row-major OCP fp8 E4M3FN bytes, one per group of 16 columns.
 *   codebook  float [16]       the 16 levels indexed by code (need not be sorted).
 *   s_channel float [N]        per-output-channel fp32 scale.
 *
 * Conventions for every entry point:
 *   - All buffers are DEVICE pointers owned by the caller, dense row-major, no strides.
 *     The library allocates, frees and retains nothing and keeps no state between
 *     calls; it never synchronises the stream.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously on it; concurrent calls on different streams are independent.
 *   - Arguments are validated on the host before anything is launched; a call that
 *     returns an error has enqueued nothing and written nothing.
 *   - Return value: W4A8_OK (0) or one of the W4A8_ERR_* codes below.  No exception
 *     crosses the ABI.  w4a8_status_string() names a code.
 *   - Alignment: x, w, xq, qpacked, srel, w8 and out must be 16-byte aligned; xs,
 *     codebook, s_channel and bias 4-byte aligned.
 *   - Sizes: M >= 0 (M == 0 is a valid call that does nothing), N >= 1,
 *     256 <= K <= W4A8_MAX_K with K % 256 == 0 (the bound keeps every int32
 *     accumulator exact: 127 * 128 * K < 2^31).
 */
#ifndef W4A8_H
#define W4A8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum w4a8_status {
    W4A8_OK = 0,
    W4A8_ERR_INVALID_ARG = 1,  /* NULL required pointer, negative size, unknown out_type */
    W4A8_ERR_SHAPE = 2,        /* N < 1, K not a positive multiple of 256, K > W4A8_MAX_K,
                                  N not a multiple of 8 for w4a8_grad_input, odd N with
                                  W4A8_OUT_SWIGLU_BF16 */
    W4A8_ERR_ALIGN = 3,        /* a pointer misses its required alignment */
    W4A8_ERR_UNSUPPORTED = 4,  /* group != 16, rot_block != 256, qmax not in 1..127,
                                  M > W4A8_GEMV_MAX_M for the GEMV entry points,
                                  K > w4a8_gemv_act_max_k(M) for w4a8_gemv_act */
    W4A8_ERR_HIP = 5           /* the HIP runtime reported an error at launch */
};

enum w4a8_out_type {
    W4A8_OUT_BF16 = 0,        /* bfloat16, round to nearest even */
    W4A8_OUT_F32 = 1,         /* float32 */
    W4A8_OUT_I32 = 2,         /* the raw int32 accumulator acc[m, n], no scaling or bias */
    W4A8_OUT_SWIGLU_BF16 = 3  /* SwiGLU fused into the epilogue (h3-rs src/weights.rs,
                                 swiglu_interleaved): the layer's rows hold gate and up
                                 projections interleaved (gate j in row 2j, up j in row
                                 2j + 1, as interleave_rows/interleave_swiglu lay them out;
                                 quantisation is row-wise, so the rows may be interleaved
                                 before or after it); out is bf16 [M, N/2] with
                                 out[m, j] = bf16(silu(y[m, 2j]) * y[m, 2j + 1]), y the fp32
                                 epilogue value and silu(g) = g / (1 + exp(-g)) in fp32.
                                 N must be even. */
};

#define W4A8_ROT_BLOCK 256
#define W4A8_GROUP 16
#define W4A8_GEMV_MAX_M 8
#define W4A8_MAX_K 131072
#define W4A8_MAX_LORA_RANK 4096

/*
 * rotate_quant_act -- steps 1 and 2 for M rows of activations.
 *
 * Follows h3-rs weights.rs fn rotate_activation (block rotation of the last dim by the
 * Kronecker-power Hadamard of fn hadamard, divided by 16 for block 256) and ai-toolkit
 * w4a8_act_quant_kernel (per-row absmax, scale = amax / qmax or 1.0 for a zero row,
 * q = round_half_even(v / scale) clamped to [-qmax, qmax]).  The division is the IEEE
 * fp32 one.  The rotated value v is the exact block product rounded once to fp32
 * whenever, in every 256-column block, E - L <= 44, with E the exponent of the largest
 * input magnitude and L the exponent of the lowest set significand bit among the
 * non-zero inputs (for bf16 this holds when every non-zero magnitude of a block lies
 * within 2^37 of the block's largest); the fp64 stages are exact there.  Blocks beyond
 * that bound get the fp64 stages' rounding (a few units of 2^-53 of the largest
 * partial sum) before the one rounding to fp32.
 * Non-finite values: a row any of whose rotated values is not finite (an inf or NaN
 * input, or a block whose product overflows fp32) gets xs = NaN and all codes 0, so
 * every output of that row in w4a8_gemm / w4a8_gemv is NaN.  w4a8_gemv_act applies
 * the same rule.
 *
 *   x         in   bf16 bits [M, K]
 *   M, K           rows and columns
 *   rot_block      must be 256
 *   qmax           1..127 (the layer uses 127)
 *   xq        out  int8 [M, K]
 *   xs        out  float [M], the per-row scales
 */
int rotate_quant_act(const void* x, int64_t M, int64_t K, int32_t rot_block, int32_t qmax,
                     int8_t* xq, float* xs, void* stream);

/*
 * decode_w4_to_int8 -- step 3 materialised: the int8 grid of a whole layer.
 *
 * ai-toolkit module docstring and unpack_w4a8_eager with W4A8_SAT:
 *   w8[n, k] = saturate_[-128,127](round_half_even(codebook[code(n, k)] * e4m3(srel[n, k/16])))
 * with the product in fp32.  A NaN scale byte (0x7F, 0xFF) decodes to 0.
 *
 *   qpacked, srel, codebook   in   the layer storage (see above)
 *   N, K                           output and input channels
 *   group                          must be 16
 *   w8                        out  int8 [N, K]
 */
int decode_w4_to_int8(const uint8_t* qpacked, const uint8_t* srel, const float* codebook,
                      int64_t N, int64_t K, int32_t group, int8_t* w8, void* stream);

/*
 * w4a8_gemm -- steps 3 to 5 for any M (the prefill path of ai-toolkit
 * _w4a8_linear_ste_op: decoded int8 grid x int8 activations -> int32 -> epilogue).
 * The weight is decoded on chip; no int8 weight copy is written to memory.
 *
 *   xq, xs              in   int8 [M, K] and float [M] from rotate_quant_act
 *   M                        rows (tokens), >= 0
 *   qpacked, srel,      in   the layer storage
 *   codebook, s_channel
 *   bias                in   float [N] or NULL
 *   N, K, group              sizes; group must be 16
 *   out_type                 W4A8_OUT_BF16, W4A8_OUT_F32, W4A8_OUT_I32 or W4A8_OUT_SWIGLU_BF16
 *   out                 out  [M, N] of the chosen type ([M, N/2] bf16 for SwiGLU)
 */
int w4a8_gemm(const int8_t* xq, const float* xs, int64_t M,
              const uint8_t* qpacked, const uint8_t* srel, const float* codebook,
              const float* s_channel, const float* bias, int64_t N, int64_t K, int32_t group,
              int32_t out_type, void* out, void* stream);

/*
 * w4a8_gemv -- the same result as w4a8_gemm for 1 <= M <= W4A8_GEMV_MAX_M, computed by
 * the decode-path kernel of ai-toolkit w4a8_gemv_kernel: packed codes, fp8 group
 * scales and the codebook are read directly and multiply-accumulated in int32 with
 * vector dot products (no matrix cores).  Output is bit-identical to w4a8_gemm.
 * M > W4A8_GEMV_MAX_M returns W4A8_ERR_UNSUPPORTED.  Arguments as for w4a8_gemm.
 */
int w4a8_gemv(const int8_t* xq, const float* xs, int64_t M,
              const uint8_t* qpacked, const uint8_t* srel, const float* codebook,
              const float* s_channel, const float* bias, int64_t N, int64_t K, int32_t group,
              int32_t out_type, void* out, void* stream);

/*
 * w4a8_gemv_act -- steps 1 to 5 in one launch for 1 <= M <= W4A8_GEMV_MAX_M: the decode
 * GEMV taking the bf16 activation rows themselves.  Every workgroup rotates and
 * quantises the M rows in on-chip memory with the arithmetic of rotate_quant_act
 * (ai-toolkit ConvRotW4A8Quantizer.forward on the decode path: prepare_act, then the
 * GEMV), so the result is bit-identical to rotate_quant_act followed by w4a8_gemv.
 *
 *   x                   in   bf16 bits [M, K]
 *   M                        rows, 0..W4A8_GEMV_MAX_M
 *   rot_block, qmax          as for rotate_quant_act
 *   qpacked, srel,      in   the layer storage
 *   codebook, s_channel
 *   bias                in   float [N] or NULL
 *   N, K, group, out_type    as for w4a8_gemm
 *   out                 out  [M, N] of the chosen type
 *   xq_out, xs_out      out  NULL, or int8 [M, K] and float [M]: the quantised rows and
 *                            their scales, as rotate_quant_act would write them (for a
 *                            caller that shares them with other layers); both or neither
 *
 * K must not exceed w4a8_gemv_act_max_k(M) (the rows are held on chip); larger K, or
 * M > W4A8_GEMV_MAX_M, returns W4A8_ERR_UNSUPPORTED.
 */
int w4a8_gemv_act(const void* x, int64_t M, int32_t rot_block, int32_t qmax,
                  const uint8_t* qpacked, const uint8_t* srel, const float* codebook,
                  const float* s_channel, const float* bias, int64_t N, int64_t K, int32_t group,
                  int32_t out_type, void* out, int8_t* xq_out, float* xs_out, void* stream);

/* Largest K that w4a8_gemv_act accepts for M rows (32768 / 16384 / 8192 / 4096 for
 * M = 1 / 2 / 3..4 / 5..8); 0 for M outside 1..W4A8_GEMV_MAX_M. */
int64_t w4a8_gemv_act_max_k(int64_t M);

/*
 * w4a8_gemv_grouped -- w4a8_gemv for several independent layers in as few launches as
 * possible (64 layers per launch): the decode path of ai-toolkit w4a8_gemv_kernel for
 * each layer, with the per-launch latency paid once per 64 layers instead of once per
 * layer.  Every layer's output is bit-identical to a w4a8_gemv call on it.
 *
 *   layers    in   HOST array of `count` descriptors (read during the call only); each
 *                  names one layer's activations (xq [M, K], xs [M]), storage, optional
 *                  bias, output [M, N] and sizes, with the same meaning and alignment
 *                  rules as the arguments of w4a8_gemv.  Outputs must not overlap.
 *   count          number of layers, >= 0 (0 does nothing)
 *   M              rows per layer, common to all layers, 0..W4A8_GEMV_MAX_M
 *   group          must be 16
 *   out_type       common output type
 * The sum of N over the layers must not exceed 2^30.  Any invalid descriptor rejects
 * the whole call before anything is launched.
 */
typedef struct w4a8_gemv_layer {
    const int8_t* xq;
    const float* xs;
    const uint8_t* qpacked;
    const uint8_t* srel;
    const float* codebook;
    const float* s_channel;
    const float* bias;   /* or NULL */
    void* out;
    int64_t N;
    int64_t K;
} w4a8_gemv_layer;

int w4a8_gemv_grouped(const w4a8_gemv_layer* layers, int32_t count, int64_t M, int32_t group,
                      int32_t out_type, void* stream);

/*
 * quantize_w4 -- the weight quantiser: an fp32 weight to the layer storage above.
 *
 * ai-toolkit ConvRotW4A8Quantizer.quantize_ (the weight is first rotated like the
 * activations, h3-rs fn hadamard with block 256, exact product rounded once to fp32)
 * and _quantize_rotated_rows with _assign_codes, grid_levels and _assign_grid:
 * per group of 16 the absmax scale, the nearest codebook level, two least-squares
 * refinements of the group scale (sums of fp32 products accumulated in column order,
 * rounded once to fp32), the channel scale max |level * scale| / 127, the fp8 e4m3
 * relative group scale (round to nearest even, above 464 -> NaN byte), and the final
 * codes as the nearest int8-grid levels of w / s_channel.  Nearest means: among the
 * two levels around the value (by the count of levels below it), the upper one only
 * if it is strictly closer.  Rows are independent; the result is deterministic.
 *
 *   w          in   float [N, K]: the weight, or the already rotated weight if rotated != 0
 *   N, K            sizes (limits as above)
 *   rot_block       must be 256
 *   group           must be 16
 *   rotated         0: rotate w first; nonzero: w is already in the rotated basis
 *   codebook   in   float [16], sorted ascending
 *   qpacked    out  uint8 [N, K/2]
 *   srel       out  uint8 [N, K/16]
 *   s_channel  out  float [N]
 * Weights must be finite.  Alignment: w 16 bytes.
 */
int quantize_w4(const float* w, int64_t N, int64_t K, int32_t rot_block, int32_t group, int32_t rotated,
                const float* codebook, uint8_t* qpacked, uint8_t* srel, float* s_channel, void* stream);

/*
 * requantize_codes_w4 -- new 4-bit codes for an fp32 weight on a layer's STORED group
 * scales, channel scales and codebook (ai-toolkit ConvRotW4A8Quantizer.requantize_codes_,
 * the grid a quantisation-aware run trains against, with _assign_grid):
 *   w_rot  = the weight rotated like quantize_w4 (unless `rotated`);
 *   target = fp32(w_rot / s_channel[n]);
 *   levels = clamp(rint(fp32(codebook[c] * e4m3(srel[n, k/16]))), -127, 127);
 *   code   = the nearest level (left insertion point p, upper candidate only if strictly
 *            closer) -- or, when u is not NULL, the unbiased stochastic choice between
 *            the bracketing levels: lo = clamp(p - 1, 0, 14),
 *            thr = fp32(fp32(u * fp32(level[lo+1] - level[lo])) + level[lo]),
 *            code = lo + (target > thr).
 * The codebook must be sorted ascending (the levels are then non-decreasing).
 *
 *   w            in   float [N, K], the weight (plain basis, or rotated if `rotated`)
 *   N, K, rot_block, group   as for quantize_w4
 *   rotated           0 or 1
 *   codebook, srel,   in   the layer's stored codebook [16], scale bytes [N, K/16] and
 *   s_channel              channel scales [N]
 *   u            in   NULL (nearest) or float [N, K] uniform draws in [0, 1) (the page
 *                     draws them with rand_like; they are inputs here)
 *   qpacked      out  uint8 [N, K/2], the new codes (the scales are not written)
 */
int requantize_codes_w4(const float* w, int64_t N, int64_t K, int32_t rot_block, int32_t group, int32_t rotated,
                        const float* codebook, const uint8_t* srel, const float* s_channel, const float* u,
                        uint8_t* qpacked, void* stream);

/*
 * fake_quant_w4 -- ai-toolkit ConvRotW4A8Quantizer.fake_quant_rotated_weight:
 * dequant(quant(w_rot)) on the stored scales, out[n, k] = fp32(level * s_channel[n])
 * with level the nearest grid level of fp32(w_rot[n, k] / s_channel[n]) (as in
 * requantize_codes_w4).
 *
 *   w_rot        in   float [N, K], the weight in the rotated basis
 *   N, K, group       sizes; group must be 16
 *   codebook, srel, s_channel   in   the layer's stored codebook, scale bytes, channel scales
 *   out          out  float [N, K] (may not overlap w_rot)
 */
int fake_quant_w4(const float* w_rot, int64_t N, int64_t K, int32_t group, const float* codebook,
                  const uint8_t* srel, const float* s_channel, float* out, void* stream);

/*
 * dequantize_w4 -- ai-toolkit dequantize_w4a8: the layer's weight in fp32,
 * out = fp32(w8 * s_channel[n]) with w8 the decoded int8 grid (as decode_w4_to_int8),
 * rotated back to the plain basis when `rotate_back` (each 256-column block times
 * H4^(x4) / 16; the exact block sum rounded once to fp32), else left rotated.
 *
 *   qpacked, srel, codebook, s_channel   in   the layer storage
 *   N, K, rot_block, group                    sizes; rot_block 256, group 16
 *   rotate_back                               0 or 1
 *   out                                  out  float [N, K]
 */
int dequantize_w4(const uint8_t* qpacked, const uint8_t* srel, const float* codebook, const float* s_channel,
                  int64_t N, int64_t K, int32_t rot_block, int32_t group, int32_t rotate_back, float* out,
                  void* stream);

/*
 * w4a8_grad_input -- the straight-through backward of the layer (ai-toolkit
 * _w4a8_linear_ste_backward): grad_x = grad @ w with
 *   w[n, k] = bf16(bf16(w8[n, k]) * bf16(s_channel[n]))      (each cast round-to-nearest-even)
 * the decoded int8 grid times the channel scale in bf16; products accumulated in fp32
 * on the matrix cores, the result rounded to bf16.  The gradient is with respect to the
 * layer's rotated input xr (the input of step 2 above), as on the page; the gradient
 * with respect to x is its block rotation (the rotation is its own inverse).  The weight
 * is decoded on chip; nothing but grad_x is written.
 *
 *   grad                in   bf16 bits [M, N], the gradient of the layer's output
 *   M                        rows, >= 0
 *   qpacked, srel,      in   the layer storage
 *   codebook, s_channel
 *   N, K, group              N must be a multiple of 8 (16-byte rows of grad); group 16
 *   out                 out  bf16 bits [M, K]
 */
int w4a8_grad_input(const void* grad, int64_t M, const uint8_t* qpacked, const uint8_t* srel,
                    const float* codebook, const float* s_channel, int64_t N, int64_t K, int32_t group,
                    void* out, void* stream);

/*
 * lora_merge_w4 -- folds one low-rank adapter into the layer's weight (h3-rs 0.2.0
 * src/weights.rs, QLinear::merge_loras: dequantise, add the delta, requantise), the
 * first two steps:
 *   out[n, k] = fp32(w[n, k] + fp32(scale * sum_r lora_b[n, r] * lora_a[r, k]))
 * with w the dequantised weight in the plain basis (as dequantize_w4 with rotate_back)
 * and the sum over r formed in fp64 in r order (each product, then each sum, rounded
 * in fp64; no fused multiply-add), times scale in fp64, rounded once to fp32.  The
 * result is the plain-basis fp32 weight that quantize_w4 (or requantize_codes_w4) turns
 * back into the layer; several adapters are merged one call at a time.
 *
 *   qpacked, srel, codebook, s_channel   in   the layer storage
 *   N, K, rot_block, group                    sizes; rot_block 256, group 16
 *   lora_a                               in   float [rank, K] (the down projection A)
 *   lora_b                               in   float [N, rank] (the up projection B)
 *   rank                                      0..W4A8_MAX_LORA_RANK (0: out is the dequantised weight)
 *   scale                                     the adapter's scale (alpha / rank, say)
 *   out                                  out  float [N, K]
 */
int lora_merge_w4(const uint8_t* qpacked, const uint8_t* srel, const float* codebook, const float* s_channel,
                  int64_t N, int64_t K, int32_t rot_block, int32_t group, const float* lora_a, const float* lora_b,
                  int32_t rank, float scale, float* out, void* stream);

/*
 * w4a8_empty_launch -- measurement aid, not a step of the layer: launches a kernel that
 * does nothing, with `blocks` workgroups of `threads` threads, on `stream`.  Timing it
 * back to back gives the launch-and-drain floor that any kernel of that grid pays, to
 * set beside the decode GEMV's duration.
 *   blocks    1 .. 2^20;  threads  64 .. 1024, a multiple of 64
 * Errors: W4A8_ERR_INVALID_ARG outside those ranges; W4A8_ERR_HIP on a launch failure.
 */
int w4a8_empty_launch(int32_t blocks, int32_t threads, void* stream);

/* Name of a status code ("W4A8_OK", ...); never NULL. */
const char* w4a8_status_string(int status);

/* ABI version of this header (incremented on any signature change). */
int w4a8_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
