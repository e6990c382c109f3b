"""Python binding of libw4a8 (the C ABI in include/w4a8.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libw4a8.so.  PyTorch supplies device memory and the current stream.  There is
no fallback: if the library is not built, or a tensor is not on the GPU, the
call raises.

    layer = W4A8Layer(qpacked, srel, codebook, s_channel, bias=None)   # device tensors
    y = linear(x_bf16, layer)               # rotate+quant, then GEMV (M <= 8) or GEMM
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a8.so")

OK, ERR_INVALID_ARG, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_HIP = range(6)
OUT_BF16, OUT_F32, OUT_I32, OUT_SWIGLU = 0, 1, 2, 3
# out_dtype value of the SwiGLU epilogue: bf16 [M, N/2] = silu(gate) * up on
# gate/up-interleaved rows
SWIGLU = "swiglu"
ROT_BLOCK, GROUP, GEMV_MAX_M, MAX_K = 256, 16, 8, 131072
ABI_VERSION = 9
FUSED_ACT_MAX_K = 4096   # linear() uses w4a8_gemv_act for one row up to this K
_OUT_CODES = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32, torch.int32: OUT_I32, SWIGLU: OUT_SWIGLU}


def _out_spec(out_dtype, m: int, n: int):
    """(shape, torch dtype) of a linear output of type out_dtype."""
    if out_dtype == SWIGLU:
        if n % 2:
            raise ValueError("the SwiGLU epilogue needs an even number of output rows")
        return (m, n // 2), torch.bfloat16
    return (m, n), out_dtype

# The default 16-level table (ai-toolkit convrot_w4a8_quant.py, FIXED_CODEBOOK):
# Lloyd-Max levels for a group-normalised Gaussian, index = 4-bit code.
FIXED_CODEBOOK = (
    -0.980602, -0.794529, -0.638165, -0.500986, -0.377321, -0.263187, -0.155210, -0.050720,
    0.052541, 0.156985, 0.265284, 0.379533, 0.502636, 0.638953, 0.794876, 0.980671,
)

# Symbols declared in include/w4a8.h, with their ctypes signatures.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
SIGNATURES = {
    "rotate_quant_act": [_P, _I64, _I64, _I32, _I32, _P, _P, _P],
    "decode_w4_to_int8": [_P, _P, _P, _I64, _I64, _I32, _P, _P],
    "w4a8_gemm": [_P, _P, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P],
    "w4a8_gemv": [_P, _P, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P],
    "quantize_w4": [_P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P],
    "w4a8_gemv_grouped": [_P, _I32, _I64, _I32, _I32, _P],
    "w4a8_gemv_act": [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P, _P, _P],
    "w4a8_gemv_act_max_k": [_I64],
    "requantize_codes_w4": [_P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P],
    "fake_quant_w4": [_P, _I64, _I64, _I32, _P, _P, _P, _P, _P],
    "dequantize_w4": [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P],
    "w4a8_grad_input": [_P, _I64, _P, _P, _P, _P, _I64, _I64, _I32, _P, _P],
    "lora_merge_w4": [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P, _I32, ctypes.c_float, _P, _P],
    "w4a8_status_string": [ctypes.c_int],
    "w4a8_abi_version": [],
    "w4a8_empty_launch": [_I32, _I32, _P],
}

_lib = None


class GemvLayerDesc(ctypes.Structure):
    """Mirror of struct w4a8_gemv_layer in include/w4a8.h."""
    _fields_ = [("xq", _P), ("xs", _P), ("qpacked", _P), ("srel", _P), ("codebook", _P), ("s_channel", _P),
                ("bias", _P), ("out", _P), ("N", _I64), ("K", _I64)]


class W4A8Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


class W4A8ArgumentError(W4A8Error, ValueError):
    pass


def load() -> ctypes.CDLL:
    """Load libw4a8.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python -m bit_codebook_quantized_amd.build` "
                              "or __graft_entry__.build() first (there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = {"w4a8_status_string": ctypes.c_char_p, "w4a8_gemv_act_max_k": ctypes.c_int64}.get(
                name, ctypes.c_int)
        if lib.w4a8_abi_version() != ABI_VERSION:
            raise ImportError("libw4a8.so ABI version mismatch")
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().w4a8_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status == OK:
        return
    if status == ERR_HIP:
        raise W4A8Error(fn, status)
    raise W4A8ArgumentError(fn, status)


def call(fn: str, *args) -> int:
    """Call a C entry point with raw arguments (pointers as ints); returns the status."""
    return getattr(load(), fn)(*args)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _out(t, shape, dtype, device, name: str) -> torch.Tensor:
    """A caller-provided output buffer must match exactly; None allocates one."""
    if t is None:
        return torch.empty(*shape, dtype=dtype, device=device)
    _dev(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


@dataclass
class W4A8Layer:
    """Device storage of one ConvRot W4A8 linear layer (see include/w4a8.h)."""
    qpacked: torch.Tensor          # uint8 [N, K/2]
    srel: torch.Tensor             # uint8 [N, K/16], fp8 e4m3fn bytes
    codebook: torch.Tensor         # float32 [16]
    s_channel: torch.Tensor        # float32 [N]
    bias: Optional[torch.Tensor] = None   # float32 [N]

    @property
    def out_features(self) -> int:
        return self.qpacked.shape[0]

    @property
    def in_features(self) -> int:
        return self.qpacked.shape[1] * 2

    @classmethod
    def from_host(cls, qpacked, srel, codebook, s_channel, bias=None, device="cuda"):
        t = lambda a, dt: torch.as_tensor(a).to(device=device, dtype=dt).contiguous()
        return cls(t(qpacked, torch.uint8), t(srel, torch.uint8), t(codebook, torch.float32),
                   t(s_channel, torch.float32), None if bias is None else t(bias, torch.float32))

    def check(self) -> None:
        n, kh = self.qpacked.shape
        _dev(self.qpacked, torch.uint8, "qpacked")
        _dev(self.srel, torch.uint8, "srel")
        _dev(self.codebook, torch.float32, "codebook")
        _dev(self.s_channel, torch.float32, "s_channel")
        if tuple(self.srel.shape) != (n, 2 * kh // GROUP) or self.codebook.numel() != 16 \
                or tuple(self.s_channel.shape) != (n,):
            raise ValueError("W4A8Layer tensor shapes do not match")
        if self.bias is not None:
            _dev(self.bias, torch.float32, "bias")
            if tuple(self.bias.shape) != (n,):
                raise ValueError("bias must be [N]")


def rotate_quant_act(x: torch.Tensor, qmax: int = 127, xq: torch.Tensor = None, xs: torch.Tensor = None):
    """bf16 x [M, K] -> (int8 xq [M, K], float32 xs [M])."""
    _dev(x, torch.bfloat16, "x")
    m, k = x.shape
    xq = _out(xq, (m, k), torch.int8, x.device, "xq")
    xs = _out(xs, (m,), torch.float32, x.device, "xs")
    _check("rotate_quant_act", load().rotate_quant_act(x.data_ptr(), m, k, ROT_BLOCK, qmax, xq.data_ptr(),
                                                      xs.data_ptr(), _stream(x)))
    return xq, xs


def decode_w4_to_int8(layer: W4A8Layer, out: torch.Tensor = None) -> torch.Tensor:
    """The layer's int8 grid [N, K]."""
    layer.check()
    n, k = layer.out_features, layer.in_features
    out = _out(out, (n, k), torch.int8, layer.qpacked.device, "out")
    _check("decode_w4_to_int8", load().decode_w4_to_int8(layer.qpacked.data_ptr(), layer.srel.data_ptr(),
                                                         layer.codebook.data_ptr(), n, k, GROUP, out.data_ptr(),
                                                         _stream(layer.qpacked)))
    return out


def _linear_call(fn: str, xq, xs, layer: W4A8Layer, out_dtype, out):
    layer.check()
    _dev(xq, torch.int8, "xq")
    _dev(xs, torch.float32, "xs")
    m, k = xq.shape
    n = layer.out_features
    if tuple(xs.shape) != (m,):
        raise ValueError(f"xs must have shape ({m},)")
    if k != layer.in_features:
        raise ValueError(f"xq has K={k}, layer has K={layer.in_features}")
    if out_dtype not in _OUT_CODES:
        raise ValueError(f"unsupported out_dtype {out_dtype}")
    shape, dt = _out_spec(out_dtype, m, n)
    out = _out(out, shape, dt, xq.device, "out")
    bias = layer.bias.data_ptr() if layer.bias is not None else None
    st = getattr(load(), fn)(xq.data_ptr(), xs.data_ptr(), m, layer.qpacked.data_ptr(), layer.srel.data_ptr(),
                             layer.codebook.data_ptr(), layer.s_channel.data_ptr(), bias, n, k, GROUP,
                             _OUT_CODES[out_dtype], out.data_ptr(), _stream(xq))
    _check(fn, st)
    return out


def w4a8_gemm(xq, xs, layer: W4A8Layer, out_dtype=torch.bfloat16, out=None):
    return _linear_call("w4a8_gemm", xq, xs, layer, out_dtype, out)


def w4a8_gemv(xq, xs, layer: W4A8Layer, out_dtype=torch.bfloat16, out=None):
    return _linear_call("w4a8_gemv", xq, xs, layer, out_dtype, out)


def gemv_act_max_k(m: int) -> int:
    """Largest K that w4a8_gemv_act takes for m rows (0 outside 1..8)."""
    return int(load().w4a8_gemv_act_max_k(int(m)))


def w4a8_gemv_act(x: torch.Tensor, layer: W4A8Layer, out_dtype=torch.bfloat16, out=None, qmax: int = 127,
                  xq_out: torch.Tensor = None, xs_out: torch.Tensor = None):
    """The whole layer for bf16 x [M, K], M <= 8, in one launch (rotation and
    quantisation done inside the GEMV).  Bit-identical to rotate_quant_act followed by
    w4a8_gemv.  xq_out / xs_out (both or neither) receive the prepared activations."""
    layer.check()
    _dev(x, torch.bfloat16, "x")
    m, k = x.shape
    n = layer.out_features
    if k != layer.in_features:
        raise ValueError(f"x has K={k}, layer has K={layer.in_features}")
    if out_dtype not in _OUT_CODES:
        raise ValueError(f"unsupported out_dtype {out_dtype}")
    if (xq_out is None) != (xs_out is None):
        raise ValueError("xq_out and xs_out go together")
    shape, dt = _out_spec(out_dtype, m, n)
    out = _out(out, shape, dt, x.device, "out")
    if xq_out is not None:
        _out(xq_out, (m, k), torch.int8, x.device, "xq_out")
        _out(xs_out, (m,), torch.float32, x.device, "xs_out")
    bias = layer.bias.data_ptr() if layer.bias is not None else None
    st = load().w4a8_gemv_act(x.data_ptr(), m, ROT_BLOCK, qmax, layer.qpacked.data_ptr(), layer.srel.data_ptr(),
                              layer.codebook.data_ptr(), layer.s_channel.data_ptr(), bias, n, k, GROUP,
                              _OUT_CODES[out_dtype], out.data_ptr(),
                              None if xq_out is None else xq_out.data_ptr(),
                              None if xs_out is None else xs_out.data_ptr(), _stream(x))
    _check("w4a8_gemv_act", st)
    return out


def _group_descs(items, out_dtype):
    """items: (xq, xs, layer, out or None) per layer, common M -> (ctypes array, outs, M)."""
    if out_dtype not in _OUT_CODES:
        raise ValueError(f"unsupported out_dtype {out_dtype}")
    arr = (GemvLayerDesc * max(len(items), 1))()
    outs, m = [], None
    for i, (xq, xs, layer, out) in enumerate(items):
        layer.check()
        _dev(xq, torch.int8, "xq")
        _dev(xs, torch.float32, "xs")
        mi, k = xq.shape
        if m is None:
            m = mi
        if mi != m or tuple(xs.shape) != (m,) or k != layer.in_features:
            raise ValueError(f"layer {i}: activations do not match (M must be common to all layers)")
        n = layer.out_features
        shape, dt = _out_spec(out_dtype, m, n)
        out = _out(out, shape, dt, xq.device, "out")
        outs.append(out)
        arr[i] = GemvLayerDesc(xq.data_ptr(), xs.data_ptr(), layer.qpacked.data_ptr(), layer.srel.data_ptr(),
                               layer.codebook.data_ptr(), layer.s_channel.data_ptr(),
                               layer.bias.data_ptr() if layer.bias is not None else None, out.data_ptr(), n, k)
    return arr, outs, (m or 0)


def w4a8_gemv_grouped(items, out_dtype=torch.bfloat16):
    """The GEMV of several independent layers, 32 per launch.  items: list of
    (xq [M, K], xs [M], W4A8Layer, out [M, N] or None) with a common M <= 8.
    Returns the outputs (bit-identical to w4a8_gemv on each layer)."""
    arr, outs, m = _group_descs(items, out_dtype)
    if items:
        _check("w4a8_gemv_grouped", load().w4a8_gemv_grouped(ctypes.addressof(arr), len(items), m, GROUP,
                                                            _OUT_CODES[out_dtype], _stream(items[0][0])))
    return outs


def prepared_gemv_grouped(items, out_dtype=torch.bfloat16):
    """prepare() for w4a8_gemv_grouped: the descriptor array is built and checked once
    (outputs given as None are allocated here, once).  The callable runs the group and
    returns the outputs; it keeps every tensor it points at alive."""
    if not items:
        raise ValueError("prepared_gemv_grouped needs at least one layer")
    arr, outs, m = _group_descs(items, out_dtype)
    c, dev, n = load().w4a8_gemv_grouped, items[0][0].device, len(items)
    code = _OUT_CODES[out_dtype]

    def run():
        st = c(ctypes.addressof(arr), n, m, GROUP, code, torch.cuda.current_stream(dev).cuda_stream)
        if st:
            _check("w4a8_gemv_grouped", st)
        return outs
    run.descs = arr                      # the descriptor array
    run.keep = (list(items), outs)       # the tensors behind its pointers
    run.outs = outs
    run()
    return run


def quantize_w4(w: torch.Tensor, codebook=None, rotated: bool = False, bias=None) -> W4A8Layer:
    """fp32 weight [N, K] on the GPU -> W4A8Layer (packed codes, fp8 group scales,
    channel scales).  ``rotated`` says the weight is already in the rotated basis.
    ``codebook`` defaults to FIXED_CODEBOOK and must be sorted ascending."""
    _dev(w, torch.float32, "w")
    n, k = w.shape
    cb = torch.tensor(FIXED_CODEBOOK if codebook is None else codebook, dtype=torch.float32, device=w.device) \
        if not isinstance(codebook, torch.Tensor) else _dev(codebook, torch.float32, "codebook")
    qp = torch.empty(n, k // 2, dtype=torch.uint8, device=w.device)
    sr = torch.empty(n, k // GROUP, dtype=torch.uint8, device=w.device)
    sch = torch.empty(n, dtype=torch.float32, device=w.device)
    _check("quantize_w4", load().quantize_w4(w.data_ptr(), n, k, ROT_BLOCK, GROUP, int(bool(rotated)), cb.data_ptr(),
                                             qp.data_ptr(), sr.data_ptr(), sch.data_ptr(), _stream(w)))
    if bias is not None:
        bias = _dev(bias, torch.float32, "bias")
    return W4A8Layer(qp, sr, cb, sch, bias)


def requantize_codes(w: torch.Tensor, layer: W4A8Layer, rotated: bool = False, u: torch.Tensor = None,
                     out: torch.Tensor = None) -> torch.Tensor:
    """New packed codes [N, K/2] for the fp32 weight w [N, K] on the layer's stored
    scales (the layer is not modified): nearest grid level, or with uniform draws
    u [N, K] in [0, 1) the unbiased stochastic choice between bracketing levels."""
    layer.check()
    _dev(w, torch.float32, "w")
    n, k = w.shape
    if (n, k) != (layer.out_features, layer.in_features):
        raise ValueError(f"w is {tuple(w.shape)}, the layer is {layer.out_features}x{layer.in_features}")
    if u is not None:
        _dev(u, torch.float32, "u")
        if tuple(u.shape) != (n, k):
            raise ValueError("u must have the weight's shape")
    out = _out(out, (n, k // 2), torch.uint8, w.device, "out")
    _check("requantize_codes_w4", load().requantize_codes_w4(
        w.data_ptr(), n, k, ROT_BLOCK, GROUP, int(bool(rotated)), layer.codebook.data_ptr(), layer.srel.data_ptr(),
        layer.s_channel.data_ptr(), None if u is None else u.data_ptr(), out.data_ptr(), _stream(w)))
    return out


def fake_quant(w_rot: torch.Tensor, layer: W4A8Layer, out: torch.Tensor = None) -> torch.Tensor:
    """dequant(quant(w_rot)) on the layer's stored scales, fp32 [N, K]."""
    layer.check()
    _dev(w_rot, torch.float32, "w_rot")
    n, k = w_rot.shape
    if (n, k) != (layer.out_features, layer.in_features):
        raise ValueError(f"w_rot is {tuple(w_rot.shape)}, the layer is {layer.out_features}x{layer.in_features}")
    out = _out(out, (n, k), torch.float32, w_rot.device, "out")
    _check("fake_quant_w4", load().fake_quant_w4(w_rot.data_ptr(), n, k, GROUP, layer.codebook.data_ptr(),
                                                 layer.srel.data_ptr(), layer.s_channel.data_ptr(), out.data_ptr(),
                                                 _stream(w_rot)))
    return out


def dequantize(layer: W4A8Layer, rotate_back: bool = True, out: torch.Tensor = None) -> torch.Tensor:
    """The layer's weight in fp32 [N, K]: w8 * s_channel, rotated back to the plain
    basis unless rotate_back is false."""
    layer.check()
    n, k = layer.out_features, layer.in_features
    out = _out(out, (n, k), torch.float32, layer.qpacked.device, "out")
    _check("dequantize_w4", load().dequantize_w4(layer.qpacked.data_ptr(), layer.srel.data_ptr(),
                                                 layer.codebook.data_ptr(), layer.s_channel.data_ptr(), n, k,
                                                 ROT_BLOCK, GROUP, int(bool(rotate_back)), out.data_ptr(),
                                                 _stream(layer.qpacked)))
    return out


def grad_input(grad: torch.Tensor, layer: W4A8Layer, out: torch.Tensor = None) -> torch.Tensor:
    """The straight-through backward: bf16 grad [M, N] -> bf16 grad_x [M, K] with respect
    to the layer's rotated input (grad @ (w8 * s_channel) in bf16, fp32 accumulation)."""
    layer.check()
    _dev(grad, torch.bfloat16, "grad")
    m, n = grad.shape
    if n != layer.out_features:
        raise ValueError(f"grad has N={n}, the layer has N={layer.out_features}")
    out = _out(out, (m, layer.in_features), torch.bfloat16, grad.device, "out")
    _check("w4a8_grad_input", load().w4a8_grad_input(grad.data_ptr(), m, layer.qpacked.data_ptr(),
                                                     layer.srel.data_ptr(), layer.codebook.data_ptr(),
                                                     layer.s_channel.data_ptr(), n, layer.in_features, GROUP,
                                                     out.data_ptr(), _stream(grad)))
    return out


def lora_merged_weight(layer: W4A8Layer, lora_a: torch.Tensor, lora_b: torch.Tensor, scale: float,
                       out: torch.Tensor = None) -> torch.Tensor:
    """The layer's plain-basis fp32 weight [N, K] with one adapter folded in:
    dequantised weight + scale * (lora_b [N, r] @ lora_a [r, K])."""
    layer.check()
    n, k = layer.out_features, layer.in_features
    _dev(lora_a, torch.float32, "lora_a")
    _dev(lora_b, torch.float32, "lora_b")
    r = lora_a.shape[0]
    if tuple(lora_a.shape) != (r, k) or tuple(lora_b.shape) != (n, r):
        raise ValueError(f"adapter shapes {tuple(lora_a.shape)}, {tuple(lora_b.shape)} do not fit {n}x{k}")
    out = _out(out, (n, k), torch.float32, layer.qpacked.device, "out")
    _check("lora_merge_w4", load().lora_merge_w4(layer.qpacked.data_ptr(), layer.srel.data_ptr(),
                                                 layer.codebook.data_ptr(), layer.s_channel.data_ptr(), n, k,
                                                 ROT_BLOCK, GROUP, lora_a.data_ptr() if r else None,
                                                 lora_b.data_ptr() if r else None, r, float(scale), out.data_ptr(),
                                                 _stream(layer.qpacked)))
    return out


def merge_lora(layer: W4A8Layer, lora_a: torch.Tensor, lora_b: torch.Tensor, scale: float) -> W4A8Layer:
    """A new layer with the adapter folded in (dequantise, add, requantise with the
    layer's codebook); the bias is kept."""
    w = lora_merged_weight(layer, lora_a, lora_b, scale)
    merged = quantize_w4(w, codebook=layer.codebook, bias=layer.bias)
    del w
    return merged


def linear(x: torch.Tensor, layer: W4A8Layer, out_dtype=torch.bfloat16) -> torch.Tensor:
    """The whole layer for bf16 x [..., K]: rotate + quantise, then the GEMV for at
    most 8 rows and the GEMM otherwise; a single row with K <= FUSED_ACT_MAX_K takes
    the one-launch w4a8_gemv_act instead (measured faster there only: every workgroup
    repeats the rotation, which costs more than the saved launch for more rows)."""
    shape = x.shape
    x2 = x.reshape(-1, shape[-1]).contiguous()
    if x2.shape[0] == 1 and x2.shape[1] <= FUSED_ACT_MAX_K:
        y = w4a8_gemv_act(x2, layer, out_dtype)
        return y.reshape(*shape[:-1], y.shape[-1])
    xq, xs = rotate_quant_act(x2)
    fn = w4a8_gemv if x2.shape[0] <= GEMV_MAX_M else w4a8_gemm
    y = fn(xq, xs, layer, out_dtype)
    return y.reshape(*shape[:-1], y.shape[-1])


def prepare(fn: str, *tensors_and_args):
    """A zero-argument callable that repeats one C entry-point call with the same
    device buffers (pointers bound once; shapes are checked by the caller's first
    regular call).  For launch loops and graph capture where per-call Python
    overhead would dominate a microsecond kernel.  Tensors are passed as pointers;
    the stream is the current stream at each call."""
    c = getattr(load(), fn)
    args = [a.data_ptr() if isinstance(a, torch.Tensor) else a for a in tensors_and_args]
    dev = next(a for a in tensors_and_args if isinstance(a, torch.Tensor)).device

    def run():
        st = c(*args, torch.cuda.current_stream(dev).cuda_stream)
        if st:
            _check(fn, st)
    run.keep = tuple(a for a in tensors_and_args if isinstance(a, torch.Tensor))   # the pointers' owners
    return run


def prepared_linear(fn: str, xq, xs, layer: W4A8Layer, out, out_dtype=None):
    """prepare() for w4a8_gemm / w4a8_gemv with the checks of a regular call done once
    (out_dtype defaults to out's dtype; pass SWIGLU for the SwiGLU epilogue)."""
    out_dtype = out.dtype if out_dtype is None else out_dtype
    _linear_call(fn, xq, xs, layer, out_dtype, out)     # validates shapes and runs once
    bias = layer.bias.data_ptr() if layer.bias is not None else None
    return prepare(fn, xq, xs, xq.shape[0], layer.qpacked, layer.srel, layer.codebook, layer.s_channel, bias,
                   layer.out_features, layer.in_features, GROUP, _OUT_CODES[out_dtype], out)


def prepared_gemv_act(x, layer: W4A8Layer, out, qmax: int = 127, out_dtype=None):
    """prepare() for w4a8_gemv_act (no prepared-activation outputs); out_dtype defaults
    to out's dtype (pass SWIGLU for the SwiGLU epilogue)."""
    out_dtype = out.dtype if out_dtype is None else out_dtype
    w4a8_gemv_act(x, layer, out_dtype, out, qmax)           # validates shapes and runs once
    bias = layer.bias.data_ptr() if layer.bias is not None else None
    return prepare("w4a8_gemv_act", x, x.shape[0], ROT_BLOCK, qmax, layer.qpacked, layer.srel, layer.codebook,
                   layer.s_channel, bias, layer.out_features, layer.in_features, GROUP, _OUT_CODES[out_dtype], out,
                   None, None)


def empty_launch(blocks: int, threads: int = 256, device="cuda") -> None:
    """Launch the library's kernel that does nothing (a launch-floor measurement aid)."""
    _check("w4a8_empty_launch", load().w4a8_empty_launch(int(blocks), int(threads),
                                                         torch.cuda.current_stream(device).cuda_stream))


def prepared_rotate_quant(x, xq, xs, qmax: int = 127):
    rotate_quant_act(x, qmax, xq, xs)                    # validates shapes and runs once
    return prepare("rotate_quant_act", x, x.shape[0], x.shape[1], ROT_BLOCK, qmax, xq, xs)
