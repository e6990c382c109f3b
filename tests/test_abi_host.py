"""Host-side tests of libw4a8: it loads, exports every function include/w4a8.h
declares, and its argument validation rejects bad calls before touching the GPU
(every call here fails validation, so nothing is launched)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def w4a8():
    from bit_codebook_quantized_amd import w4a8 as b
    b.load()
    return b


def test_header_declares_the_operations():
    names = _declared_functions()
    for n in ("rotate_quant_act", "decode_w4_to_int8", "w4a8_gemm", "w4a8_gemv", "w4a8_gemv_grouped",
              "quantize_w4", "w4a8_gemv_act", "w4a8_gemv_act_max_k", "requantize_codes_w4", "fake_quant_w4",
              "dequantize_w4", "w4a8_grad_input", "lora_merge_w4", "w4a8_status_string", "w4a8_abi_version",
              "w4a8_empty_launch"):
        assert n in names
    assert len(names) == 16, names


def test_library_exports_every_declared_symbol(w4a8):
    lib = ctypes.CDLL(w4a8.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(w4a8.SIGNATURES)


def test_status_strings(w4a8):
    assert [w4a8.status_string(i) for i in range(6)] == [
        "W4A8_OK", "W4A8_ERR_INVALID_ARG", "W4A8_ERR_SHAPE", "W4A8_ERR_ALIGN", "W4A8_ERR_UNSUPPORTED",
        "W4A8_ERR_HIP"]
    assert w4a8.status_string(99) == "W4A8_ERR_UNKNOWN"
    assert w4a8.load().w4a8_abi_version() == w4a8.ABI_VERSION == 9


def test_empty_launch_rejects_bad_grids(w4a8):
    # validation happens before any HIP call, so this runs without a GPU
    for blocks, threads in [(0, 256), (-1, 64), ((1 << 20) + 1, 64), (4, 32), (4, 100), (4, 2048)]:
        assert w4a8.call("w4a8_empty_launch", blocks, threads, None) == w4a8.ERR_INVALID_ARG


A = 1 << 20          # a 16-byte-aligned fake address (never dereferenced: validation fails first)
U = A + 1            # misaligned


def _lin(w4a8, fn, **kw):
    a = dict(xq=A, xs=A, M=4, qp=A, srel=A, cb=A, sch=A, bias=None, N=64, K=256, group=16, out_type=0, out=A)
    a.update(kw)
    return w4a8.call(fn, a["xq"], a["xs"], a["M"], a["qp"], a["srel"], a["cb"], a["sch"], a["bias"], a["N"],
                     a["K"], a["group"], a["out_type"], a["out"], None)


@pytest.mark.parametrize("fn", ["w4a8_gemm", "w4a8_gemv"])
def test_linear_validation(w4a8, fn):
    assert _lin(w4a8, fn, M=-1) == w4a8.ERR_INVALID_ARG
    assert _lin(w4a8, fn, N=0) == w4a8.ERR_SHAPE
    assert _lin(w4a8, fn, N=-3) == w4a8.ERR_INVALID_ARG
    for k in (0, 128, 300, 131072 + 256):
        assert _lin(w4a8, fn, K=k) == w4a8.ERR_SHAPE, k
    assert _lin(w4a8, fn, K=-256) == w4a8.ERR_INVALID_ARG
    assert _lin(w4a8, fn, group=32) == w4a8.ERR_UNSUPPORTED
    assert _lin(w4a8, fn, out_type=4) == w4a8.ERR_INVALID_ARG
    assert _lin(w4a8, fn, out_type=3, N=63) == w4a8.ERR_SHAPE          # SwiGLU pairs rows
    assert _lin(w4a8, fn, out_type=3, M=0) == w4a8.OK
    for p in ("qp", "srel", "cb", "sch"):
        assert _lin(w4a8, fn, **{p: None}) == w4a8.ERR_INVALID_ARG, p
    for p in ("xq", "xs", "out"):
        assert _lin(w4a8, fn, **{p: None}) == w4a8.ERR_INVALID_ARG, p
        assert _lin(w4a8, fn, M=0, **{p: None, "qp": U}) == w4a8.ERR_ALIGN   # shapes ok, storage misaligned
    for p in ("xq", "qp", "srel", "out"):
        assert _lin(w4a8, fn, **{p: A + 8}) == w4a8.ERR_ALIGN, p
    for p in ("xs", "cb", "sch", "bias"):
        assert _lin(w4a8, fn, **{p: A + 2}) == w4a8.ERR_ALIGN, p


def test_gemv_rejects_more_than_8_rows(w4a8):
    assert _lin(w4a8, "w4a8_gemv", M=9) == w4a8.ERR_UNSUPPORTED
    assert _lin(w4a8, "w4a8_gemv", M=9, qp=U) == w4a8.ERR_ALIGN      # validation order: storage first
    assert _lin(w4a8, "w4a8_gemv", M=9, K=100) == w4a8.ERR_SHAPE
    assert _lin(w4a8, "w4a8_gemv", M=9, group=8) == w4a8.ERR_UNSUPPORTED


def _act(w4a8, **kw):
    a = dict(x=A, M=4, rot=256, qmax=127, qp=A, srel=A, cb=A, sch=A, bias=None, N=64, K=256, group=16, out_type=0,
             out=A, xq_out=None, xs_out=None)
    a.update(kw)
    return w4a8.call("w4a8_gemv_act", a["x"], a["M"], a["rot"], a["qmax"], a["qp"], a["srel"], a["cb"], a["sch"],
                     a["bias"], a["N"], a["K"], a["group"], a["out_type"], a["out"], a["xq_out"], a["xs_out"], None)


def test_gemv_act_validation(w4a8):
    assert [w4a8.gemv_act_max_k(m) for m in range(10)] == [0, 32768, 16384, 8192, 8192, 4096, 4096, 4096, 4096, 0]
    assert _act(w4a8, M=-1) == w4a8.ERR_INVALID_ARG
    assert _act(w4a8, M=9) == w4a8.ERR_UNSUPPORTED
    assert _act(w4a8, M=5, K=4096 + 256) == w4a8.ERR_UNSUPPORTED     # rows do not fit on chip
    assert _act(w4a8, M=1, K=32768 + 256) == w4a8.ERR_UNSUPPORTED
    assert _act(w4a8, N=0) == w4a8.ERR_SHAPE
    assert _act(w4a8, K=300) == w4a8.ERR_SHAPE
    assert _act(w4a8, rot=128) == w4a8.ERR_UNSUPPORTED
    assert _act(w4a8, qmax=0) == w4a8.ERR_UNSUPPORTED
    assert _act(w4a8, qmax=128) == w4a8.ERR_UNSUPPORTED
    assert _act(w4a8, group=32) == w4a8.ERR_UNSUPPORTED
    assert _act(w4a8, out_type=4) == w4a8.ERR_INVALID_ARG
    assert _act(w4a8, out_type=3, N=63) == w4a8.ERR_SHAPE
    for p in ("x", "out", "qp", "srel", "cb", "sch"):
        assert _act(w4a8, **{p: None}) == w4a8.ERR_INVALID_ARG, p
    assert _act(w4a8, xq_out=A) == w4a8.ERR_INVALID_ARG                # one of the pair
    assert _act(w4a8, xs_out=A) == w4a8.ERR_INVALID_ARG
    for p in ("x", "out", "qp", "srel", "xq_out"):
        kw = {"xq_out": A, "xs_out": A}
        kw[p] = A + 8
        assert _act(w4a8, **kw) == w4a8.ERR_ALIGN, p
    assert _act(w4a8, xq_out=A, xs_out=A + 2) == w4a8.ERR_ALIGN
    assert _act(w4a8, M=0, x=None, out=None, qp=U) == w4a8.ERR_ALIGN


def test_regrid_validation(w4a8):
    def rq(**kw):
        a = dict(w=A, N=4, K=256, rot=256, group=16, rotated=0, cb=A, srel=A, sch=A, u=None, out=A)
        a.update(kw)
        return w4a8.call("requantize_codes_w4", a["w"], a["N"], a["K"], a["rot"], a["group"], a["rotated"], a["cb"],
                         a["srel"], a["sch"], a["u"], a["out"], None)

    def fq(**kw):
        a = dict(w=A, N=4, K=256, group=16, cb=A, srel=A, sch=A, out=A)
        a.update(kw)
        return w4a8.call("fake_quant_w4", a["w"], a["N"], a["K"], a["group"], a["cb"], a["srel"], a["sch"], a["out"],
                         None)

    def dq(**kw):
        a = dict(qp=A, srel=A, cb=A, sch=A, N=4, K=256, rot=256, group=16, back=1, out=A)
        a.update(kw)
        return w4a8.call("dequantize_w4", a["qp"], a["srel"], a["cb"], a["sch"], a["N"], a["K"], a["rot"], a["group"],
                         a["back"], a["out"], None)

    for f in (rq, fq, dq):
        assert f(N=0) == w4a8.ERR_SHAPE
        assert f(N=-1) == w4a8.ERR_INVALID_ARG
        assert f(K=300) == w4a8.ERR_SHAPE
        assert f(group=32) == w4a8.ERR_UNSUPPORTED
        assert f(cb=None) == w4a8.ERR_INVALID_ARG
        assert f(sch=A + 2) == w4a8.ERR_ALIGN
        assert f(out=A + 8) == w4a8.ERR_ALIGN
        assert f(N=1 << 30, K=131072) == w4a8.ERR_SHAPE       # more row chunks than a grid holds
    assert rq(rot=128) == w4a8.ERR_UNSUPPORTED and dq(rot=128) == w4a8.ERR_UNSUPPORTED
    assert rq(rotated=2) == w4a8.ERR_INVALID_ARG and dq(back=2) == w4a8.ERR_INVALID_ARG
    assert rq(u=A + 4) == w4a8.ERR_ALIGN and rq(w=A + 4) == w4a8.ERR_ALIGN and fq(w=A + 4) == w4a8.ERR_ALIGN
    assert rq(w=None) == w4a8.ERR_INVALID_ARG and fq(w=None) == w4a8.ERR_INVALID_ARG and dq(qp=None) == w4a8.ERR_INVALID_ARG


def test_grad_input_validation(w4a8):
    def gi(**kw):
        a = dict(g=A, M=4, qp=A, srel=A, cb=A, sch=A, N=64, K=256, group=16, out=A)
        a.update(kw)
        return w4a8.call("w4a8_grad_input", a["g"], a["M"], a["qp"], a["srel"], a["cb"], a["sch"], a["N"], a["K"],
                         a["group"], a["out"], None)

    assert gi(M=-1) == w4a8.ERR_INVALID_ARG
    assert gi(N=60) == w4a8.ERR_SHAPE                 # rows of grad must be 16-byte multiples
    assert gi(N=0) == w4a8.ERR_SHAPE and gi(K=300) == w4a8.ERR_SHAPE
    assert gi(group=32) == w4a8.ERR_UNSUPPORTED
    for p in ("qp", "srel", "cb", "sch", "g", "out"):
        assert gi(**{p: None}) == w4a8.ERR_INVALID_ARG, p
    for p in ("g", "out", "qp", "srel"):
        assert gi(**{p: A + 8}) == w4a8.ERR_ALIGN, p
    assert gi(M=0, g=None, out=None, qp=U) == w4a8.ERR_ALIGN


def test_lora_merge_validation(w4a8):
    def lm(**kw):
        a = dict(qp=A, srel=A, cb=A, sch=A, N=8, K=256, rot=256, group=16, la=A, lb=A, r=4, scale=0.5, out=A)
        a.update(kw)
        return w4a8.call("lora_merge_w4", a["qp"], a["srel"], a["cb"], a["sch"], a["N"], a["K"], a["rot"], a["group"],
                         a["la"], a["lb"], a["r"], a["scale"], a["out"], None)

    assert lm(r=-1) == w4a8.ERR_INVALID_ARG
    assert lm(r=4097) == w4a8.ERR_UNSUPPORTED
    assert lm(la=None) == w4a8.ERR_INVALID_ARG and lm(lb=None) == w4a8.ERR_INVALID_ARG
    assert lm(r=0, la=None, lb=None, out=A + 8) == w4a8.ERR_ALIGN       # rank 0 needs no adapter
    assert lm(la=A + 4) == w4a8.ERR_ALIGN and lm(lb=A + 2) == w4a8.ERR_ALIGN
    assert lm(K=300) == w4a8.ERR_SHAPE and lm(N=0) == w4a8.ERR_SHAPE
    assert lm(rot=128) == w4a8.ERR_UNSUPPORTED and lm(group=8) == w4a8.ERR_UNSUPPORTED
    assert lm(qp=None) == w4a8.ERR_INVALID_ARG


def test_rotate_quant_validation(w4a8):
    c = lambda **kw: w4a8.call("rotate_quant_act", kw.get("x", A), kw.get("M", 4), kw.get("K", 256),
                               kw.get("rot", 256), kw.get("qmax", 127), kw.get("xq", A), kw.get("xs", A), None)
    assert c(M=-1) == w4a8.ERR_INVALID_ARG
    assert c(K=255) == w4a8.ERR_SHAPE
    assert c(rot=128) == w4a8.ERR_UNSUPPORTED
    assert c(qmax=0) == w4a8.ERR_UNSUPPORTED and c(qmax=128) == w4a8.ERR_UNSUPPORTED
    assert c(x=None) == w4a8.ERR_INVALID_ARG and c(xs=None) == w4a8.ERR_INVALID_ARG
    assert c(x=A + 2) == w4a8.ERR_ALIGN and c(xq=A + 4) == w4a8.ERR_ALIGN and c(xs=A + 1) == w4a8.ERR_ALIGN
    assert c(M=0, x=None, xq=None, xs=None) == w4a8.OK        # M == 0 is a no-op


def test_decode_validation(w4a8):
    c = lambda **kw: w4a8.call("decode_w4_to_int8", kw.get("qp", A), kw.get("srel", A), kw.get("cb", A),
                               kw.get("N", 8), kw.get("K", 256), kw.get("group", 16), kw.get("w8", A), None)
    assert c(N=0) == w4a8.ERR_SHAPE and c(K=16) == w4a8.ERR_SHAPE
    assert c(group=64) == w4a8.ERR_UNSUPPORTED
    assert c(w8=None) == w4a8.ERR_INVALID_ARG
    assert c(w8=A + 4) == w4a8.ERR_ALIGN and c(srel=A + 8) == w4a8.ERR_ALIGN


def test_quantize_validation(w4a8):
    c = lambda **kw: w4a8.call("quantize_w4", kw.get("w", A), kw.get("N", 8), kw.get("K", 256), kw.get("rot", 256),
                               kw.get("group", 16), kw.get("rotated", 0), kw.get("cb", A), kw.get("qp", A),
                               kw.get("srel", A), kw.get("sch", A), None)
    assert c(N=0) == w4a8.ERR_SHAPE and c(N=-1) == w4a8.ERR_INVALID_ARG
    assert c(K=272) == w4a8.ERR_SHAPE and c(K=-256) == w4a8.ERR_INVALID_ARG
    assert c(rot=64) == w4a8.ERR_UNSUPPORTED and c(group=32) == w4a8.ERR_UNSUPPORTED
    for p in ("w", "cb", "qp", "srel", "sch"):
        assert c(**{p: None}) == w4a8.ERR_INVALID_ARG, p
    assert c(w=A + 4) == w4a8.ERR_ALIGN and c(qp=A + 8) == w4a8.ERR_ALIGN and c(srel=A + 1) == w4a8.ERR_ALIGN
    assert c(cb=A + 2) == w4a8.ERR_ALIGN and c(sch=A + 2) == w4a8.ERR_ALIGN


def test_gemv_grouped_validation(w4a8):
    def desc(**kw):
        d = dict(xq=A, xs=A, qpacked=A, srel=A, codebook=A, s_channel=A, bias=None, out=A, N=64, K=256)
        d.update(kw)
        return w4a8.GemvLayerDesc(**d)

    def c(descs, count=None, M=1, group=16, out_type=0):
        arr = (w4a8.GemvLayerDesc * max(len(descs), 1))(*descs)
        return w4a8.call("w4a8_gemv_grouped", ctypes.addressof(arr), len(descs) if count is None else count, M,
                         group, out_type, None)
    assert ctypes.sizeof(w4a8.GemvLayerDesc) == 80
    assert c([]) == w4a8.OK and c([desc()], M=0) == w4a8.OK and c([desc()], count=0) == w4a8.OK
    assert c([desc()], count=-1) == w4a8.ERR_INVALID_ARG and c([desc()], M=-1) == w4a8.ERR_INVALID_ARG
    assert c([desc()], M=9) == w4a8.ERR_UNSUPPORTED and c([desc()], group=8) == w4a8.ERR_UNSUPPORTED
    assert c([desc()], out_type=5) == w4a8.ERR_INVALID_ARG
    assert w4a8.call("w4a8_gemv_grouped", None, 2, 1, 16, 0, None) == w4a8.ERR_INVALID_ARG
    # one bad descriptor among good ones rejects the whole call
    assert c([desc(), desc(K=300), desc()]) == w4a8.ERR_SHAPE
    assert c([desc(), desc(out=A + 8)]) == w4a8.ERR_ALIGN
    assert c([desc(), desc(srel=None)]) == w4a8.ERR_INVALID_ARG
    assert c([desc(N=1 << 29), desc(N=(1 << 29) + 1)]) == w4a8.ERR_SHAPE      # total rows above 2^30


def test_binding_rejects_cpu_tensors(w4a8):
    import torch
    with pytest.raises(ValueError):
        w4a8.rotate_quant_act(torch.zeros(2, 256, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        w4a8.quantize_w4(torch.zeros(2, 256, dtype=torch.float32))


def test_binding_default_codebook_matches_the_page_table():
    import numpy as np
    import oracle as O
    from bit_codebook_quantized_amd.w4a8 import FIXED_CODEBOOK
    assert np.array_equal(np.array(FIXED_CODEBOOK, np.float32), O.FIXED_CODEBOOK)
