"""GPU parity: every entry point of libw4a8 (called through the C ABI binding)
against the CPU oracle on the same seeded inputs.

Bar: bit-exact for the int8 grid, the int8 activations and their fp32 scales,
the int32 accumulators and the bf16 / fp32 outputs (both sides round the same
fp32 operations in the same order).  The end-to-end output is additionally held
to the 1e-3 max-abs-rel tolerance (max |y - r| / max |r|).  Small shapes cover
several tiles plus ragged tails; the full benchmark shapes are checked on
sampled rows the oracle can afford."""

import functools

import numpy as np
import pytest
import torch

import oracle as O
from bit_codebook_quantized_amd import synth
from bit_codebook_quantized_amd import w4a8 as B

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def bf16_dev(x_f32):
    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16).to(DEV)


def host_layer(packed, srel, sch, cb, bias=None):
    return B.W4A8Layer.from_host(packed, srel, cb, sch, bias)


@functools.lru_cache(maxsize=None)
def quantized_layer(n, k, config, layer=0):
    """Oracle-quantised seeded Gaussian weight (std 0.02), rotation 256, group 16."""
    w = synth.gaussian_weight(n, k, seed=synth.seed_for(config, layer, synth.ROLE_WEIGHT))
    packed, srel, sch, cb = O.quantize_w4(w)
    return packed, srel, sch, cb


@functools.lru_cache(maxsize=None)
def random_layer(n, k, seed, lo=0x00, hi=0xFF):
    return synth.random_layer_bytes(n, k, seed=seed, srel_lo=lo, srel_hi=hi)


def random_xq(m, k, seed):
    g = synth.rng(seed)
    xq = g.integers(-127, 128, size=(m, k), dtype=np.int64).astype(np.int8)
    xs = g.uniform(0.01, 0.1, size=m).astype(np.float32)
    return xq, xs


def max_abs_rel(y, r):
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    return np.abs(y - r).max() / max(np.abs(r).max(), 1e-30)


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ------------------------------------------------------------------------- decode

def test_decode_every_scale_byte_and_code():
    # row b uses scale byte b in every group; codes cycle so each group sees all 16 codes
    k = 512
    codes = (np.arange(k)[None, :] + np.arange(256)[:, None]) % 16
    packed = O.pack_codes(codes)
    srel = np.repeat(np.arange(256, dtype=np.uint8)[:, None], k // 16, axis=1)
    rng = np.random.default_rng(0)
    books = {"fixed": O.FIXED_CODEBOOK, "uniform": O.uniform_codebook(),
             "wide_unsorted": rng.uniform(-3, 3, 16).astype(np.float32)}
    for name, cb in books.items():
        say("decode all (byte, code) pairs", name)
        layer = host_layer(packed, srel, np.ones(256, np.float32), cb)
        got = B.decode_w4_to_int8(layer).cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(got, O.decode_w4(packed, srel, cb)), name


@pytest.mark.parametrize("n,k", [(1, 256), (37, 768), (300, 4096), (4096, 4096), (12288, 3072), (3, 131072)])
def test_decode_random_layers(n, k):
    say("decode random layer", n, k)
    packed, srel, sch = random_layer(n, k, seed=1000 + n)
    layer = host_layer(packed, srel, sch, O.FIXED_CODEBOOK)
    got = B.decode_w4_to_int8(layer).cpu().numpy()
    assert np.array_equal(got, O.decode_w4(packed, srel, O.FIXED_CODEBOOK))


# ------------------------------------------------------------- rotate + quantise

RQ_CASES = [
    (16, 256, "normal"), (1, 4096, "normal"), (3, 4096, "normal"), (8, 4096, "outliers"),
    (37, 768, "student_t"), (33, 512, "normal"), (5, 1280, "normal"), (64, 3072, "student_t"),
    (5, 12288, "outliers"), (3, 8192, "normal"), (2, 36864, "student_t"), (17, 4352, "normal"),
    # a full round of blocks and a ragged last one (1, 1 and 4 rows per block)
    (2049, 4096, "outliers"), (2051, 3072, "student_t"), (8202, 1024, "normal"),
]


@pytest.mark.parametrize("m,k,kind", RQ_CASES)
def test_rotate_quant_act_bit_exact(m, k, kind):
    say("rotate_quant_act", m, k, kind)
    x = synth.activations(m, k, seed=synth.seed_for(9, m, k), kind=kind)
    if m >= 3:
        x[1] = 0.0                      # an all-zero row: scale 1, codes 0
        x[2] = 0.0
        x[2, 7] = -3.0                  # a single non-zero value
    xq, xs = B.rotate_quant_act(bf16_dev(x))
    ref_q, ref_s = O.rotate_quant_act(x)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), ref_q)


def test_rotate_quant_act_full_size_rows_with_non_finite_values():
    # the prefill activation shape with rows poisoned by an Inf or a NaN next to finite rows
    m, k = 2048, 4096
    x = synth.activations(m, k, seed=synth.seed_for(9, 7, 7), kind="normal")
    x[4, 100] = np.inf
    x[5, 3000] = np.nan
    x[1001, 0] = -np.inf
    say("rotate_quant_act full size, non-finite rows")
    xq, xs = B.rotate_quant_act(bf16_dev(x))
    rq, rs = O.rotate_quant_act(x)
    got_s = xs.cpu().numpy()
    assert np.array_equal(np.isnan(got_s), np.isnan(rs))
    fin = ~np.isnan(rs)
    assert np.array_equal(got_s[fin].view(np.uint32), rs[fin].view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), rq)


def test_rotate_quant_act_qmax_and_empty():
    x = synth.activations(4, 1024, seed=77)
    for qmax in (1, 7, 100):
        say("rotate_quant_act qmax", qmax)
        xq, xs = B.rotate_quant_act(bf16_dev(x), qmax=qmax)
        rq, rs = O.rotate_quant_act(x, qmax=qmax)
        assert np.array_equal(xq.cpu().numpy(), rq) and np.array_equal(xs.cpu().numpy(), rs)
    xq, xs = B.rotate_quant_act(torch.zeros(0, 512, dtype=torch.bfloat16, device=DEV))
    assert xq.shape == (0, 512)


def test_rotate_quant_act_extreme_magnitudes():
    # rows whose rotated values and scale are fp32 subnormals (a lone smallest bf16
    # subnormal gives a scale a few dozen subnormal steps wide, so some quotients land
    # well above qmax and only the clamp brings them back), and a row near the top of
    # the range; every code and scale must still match the oracle
    x = synth.activations(5, 1024, seed=79)
    x[0] *= 1e-38
    x[1] *= 3e-40
    x[2] *= 1e36
    x[3] = 0.0
    x[3, 300] = 9.2e-41                 # rounds to the smallest bf16 subnormal, 2^-133
    x[4] = 0.0
    x[4, 5] = -9.2e-41
    x[4, 700] = 3 * 9.2e-41
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()   # the bf16 inputs both sides see
    for qmax in (127, 7):
        say("rotate_quant_act extreme magnitudes, qmax", qmax)
        xq, xs = B.rotate_quant_act(bf16_dev(x), qmax=qmax)
        rq, rs = O.rotate_quant_act(x, qmax=qmax)
        assert np.array_equal(xs.cpu().numpy().view(np.uint32), rs.view(np.uint32))
        assert np.array_equal(xq.cpu().numpy(), rq)


def _bf16_exact(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("spread", [30, 37, 44])
def test_rotate_quant_act_at_the_exactness_bound(spread):
    # every 256-column block spans `spread` binades from the exponent of its largest input
    # (E = 0) to the lowest set significand bit of its smallest (2^-spread); up to 44 every
    # fp64 partial sum of the rotation is exact, so the result is the exact block product
    # rounded once, as the oracle forms it with integers where fp64 would not be exact
    rng = synth.rng(300 + spread)
    m, k = 6, 1024
    x = (rng.standard_normal((m, k)) * 0.25).astype(np.float32)
    x[np.abs(x) < 2.0 ** -20] = 0.0
    x = _bf16_exact(x)
    x[:, 0::256] = 1.9921875
    x[:, 1::256] = np.float32(2.0 ** -spread)
    x[:, 2::256] = -np.float32(3.0 * 2.0 ** -spread)
    x[3, 256:512] = 0.0
    x[3, 300] = np.float32(2.0 ** -spread)          # a block holding only the smallest value
    say("rotate_quant_act exactness bound, spread", spread)
    xq, xs = B.rotate_quant_act(bf16_dev(x))
    rq, rs = O.rotate_quant_act(x)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), rq)


def _non_finite_rows(m, k, seed):
    x = synth.activations(m, k, seed=seed)
    h0 = np.sign(O.hadamard(256)[0]).astype(np.float32)
    x[1, 5] = np.inf
    x[2, k - 3] = -np.inf
    x[3, 300 % k] = np.nan
    x[4, :256] = h0 * np.float32(3.3895313892515355e38)   # the largest bf16: its block overflows fp32
    x[5, 3] = np.inf
    x[5, 9] = -np.inf
    return x


def test_rotate_quant_act_rows_with_non_finite_values():
    # a row holding an inf or NaN input, or a block whose rotated value overflows fp32, has
    # no finite maximum: scale NaN and every code 0 (the oracle's reading); other rows as usual
    for m, k in [(8, 1024), (16, 256), (3, 8192), (7, 40960)]:
        x = _non_finite_rows(max(m, 6), k, seed=91 + k)
        say("rotate_quant_act non-finite rows", x.shape)
        xq, xs = B.rotate_quant_act(bf16_dev(x))
        rq, rs = O.rotate_quant_act(x)
        assert np.array_equal(xs.cpu().numpy().view(np.uint32), rs.view(np.uint32))
        assert np.array_equal(xq.cpu().numpy(), rq)
        assert np.all(np.isnan(rs[1:6])) and np.all(rq[1:6] == 0)


def test_layer_outputs_of_non_finite_rows_are_nan():
    # through the whole layer: the poisoned rows' outputs are NaN (0 * NaN scale), the other
    # rows are bit-exact; GEMM (12 rows), GEMV and the one-launch GEMV (6 rows)
    packed, srel, sch, cb = quantized_layer(384, 1024, config=9)
    layer = host_layer(packed, srel, sch, cb)
    for m in (12, 6):
        x = _non_finite_rows(m, 1024, seed=97)
        ref, *_ = O.linear(x, packed, srel, sch, cb, out="bf16")
        say("layer with non-finite rows, M =", m)
        y = bf16_bits(B.linear(bf16_dev(x), layer))
        assert np.array_equal(y, ref)
        if m <= 8:
            xq_o = torch.empty(m, 1024, dtype=torch.int8, device=DEV)
            xs_o = torch.empty(m, dtype=torch.float32, device=DEV)
            y2 = bf16_bits(B.w4a8_gemv_act(bf16_dev(x), layer, xq_out=xq_o, xs_out=xs_o))
            assert np.array_equal(y2, ref)
            rq, rs = O.rotate_quant_act(x)
            assert np.array_equal(xs_o.cpu().numpy().view(np.uint32), rs.view(np.uint32))
            assert np.array_equal(xq_o.cpu().numpy(), rq)
        assert np.all(np.isnan(O.bf16_bits_to_f32(ref[1:6])))


# ------------------------------------------------------------- integer contraction

# (256, 256, 256) and (513, 384, 1024): whole 256 x 128 tiles (their bf16 output goes through
# LDS); (512, 260, 512): whole tiles with rows that are not 16-byte aligned (direct stores);
# (1300, 512, 256): 6 x 4 tiles, so the tile order has a band of 4 row tiles and a short
# band of 2 (and 24 tiles take the XCD grouping).  K sets the number of 128-deep stages of
# the software pipeline: 2, 4, 6 (a 4-stage group and a 2-stage tail), 10, 12 and 18 (a
# first group, steady groups with constant wait counts, a last group and a tail), 24 (one
# 12-stage steady body with constant buffers, then a steady 4-stage group), 32 (two 12-stage
# bodies), 36 (two bodies, a steady group, a last group) and 42 (two bodies, two steady
# groups, a last group and a tail).
GEMM_SHAPES = [(16, 256, 256), (37, 200, 768), (300, 1000, 512), (257, 129, 256), (1, 128, 4096),
               (9, 64, 256), (513, 384, 1024), (64, 4096, 3072), (256, 256, 256), (512, 260, 512),
               (1300, 512, 256), (300, 384, 1280), (513, 260, 1536), (200, 256, 2304),
               (257, 129, 4608), (130, 300, 5376)]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_int32_exact_and_epilogue_bitwise(m, n, k):
    say("gemm", m, n, k)
    xq, xs = random_xq(m, k, seed=m * 7 + k)
    packed, srel, sch = random_layer(n, k, seed=n * 11 + k, lo=0x50, hi=0x7E)
    bias = synth.rng(n).standard_normal(n).astype(np.float32)
    w8 = O.decode_w4(packed, srel, O.FIXED_CODEBOOK)
    acc = O.gemm_exact(xq, w8)
    dxq, dxs = torch.from_numpy(xq).to(DEV), torch.from_numpy(xs).to(DEV)
    layer = host_layer(packed, srel, sch, O.FIXED_CODEBOOK)
    got = B.w4a8_gemm(dxq, dxs, layer, torch.int32).cpu().numpy()
    assert np.array_equal(got, acc)
    y32 = B.w4a8_gemm(dxq, dxs, layer, torch.float32).cpu().numpy()
    assert np.array_equal(y32.view(np.uint32), O.epilogue(acc, xs, sch, out="f32").view(np.uint32))
    layer_b = host_layer(packed, srel, sch, O.FIXED_CODEBOOK, bias)
    yb = bf16_bits(B.w4a8_gemm(dxq, dxs, layer_b, torch.bfloat16))
    assert np.array_equal(yb, O.epilogue(acc, xs, sch, bias, out="bf16"))


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8])
# K = 768, 1536, 3072 and (M <= 2) 9216 take 3 groups per lane and batch, the others 4;
# 9216 and 12288 span several activation slabs for the larger M
@pytest.mark.parametrize("n,k", [(4096, 4096), (37, 256), (257, 768), (64, 1536), (1000, 3072), (300, 9216),
                                 (130, 12288)])
def test_gemv_exact_and_equal_to_gemm(m, n, k):
    say("gemv", m, n, k)
    xq, xs = random_xq(m, k, seed=100 + m + k)
    packed, srel, sch = random_layer(n, k, seed=n + 5 * k, lo=0x50, hi=0x7E)
    bias = synth.rng(n + 1).standard_normal(n).astype(np.float32)
    acc = O.gemm_exact(xq, O.decode_w4(packed, srel, O.FIXED_CODEBOOK))
    dxq, dxs = torch.from_numpy(xq).to(DEV), torch.from_numpy(xs).to(DEV)
    layer = host_layer(packed, srel, sch, O.FIXED_CODEBOOK, bias)
    assert np.array_equal(B.w4a8_gemv(dxq, dxs, layer, torch.int32).cpu().numpy(), acc)
    yv = bf16_bits(B.w4a8_gemv(dxq, dxs, layer, torch.bfloat16))
    assert np.array_equal(yv, O.epilogue(acc, xs, sch, bias, out="bf16"))
    ym = bf16_bits(B.w4a8_gemm(dxq, dxs, layer, torch.bfloat16))
    assert np.array_equal(yv, ym)                      # decode path == prefill path, bit for bit
    yf = B.w4a8_gemv(dxq, dxs, layer, torch.float32).cpu().numpy()
    assert np.array_equal(yf.view(np.uint32), O.epilogue(acc, xs, sch, bias, out="f32").view(np.uint32))


def test_gemv_rejects_nine_rows_and_allows_zero():
    packed, srel, sch = random_layer(64, 256, seed=3)
    layer = host_layer(packed, srel, sch, O.FIXED_CODEBOOK)
    xq = torch.zeros(9, 256, dtype=torch.int8, device=DEV)
    xs = torch.ones(9, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        B.w4a8_gemv(xq, xs, layer)
    assert B.w4a8_gemv(xq[:0], xs[:0], layer).shape == (0, 64)
    assert B.w4a8_gemm(xq[:0], xs[:0], layer).shape == (0, 64)


# ---------------------------------------------------------------- end to end

def _end_to_end(x, layer_np, rows=None, label=""):
    packed, srel, sch, cb = layer_np
    layer = host_layer(packed, srel, sch, cb)
    say("end-to-end", label, x.shape)
    y = bf16_bits(B.linear(bf16_dev(x), layer))
    torch.cuda.synchronize()
    xs_rows = x if rows is None else x[rows]
    ref, _, _, _ = O.linear(xs_rows, packed, srel, sch, cb, out="bf16")
    got = y if rows is None else y[rows]
    err = max_abs_rel(O.bf16_bits_to_f32(got), O.bf16_bits_to_f32(ref))
    assert err <= 1e-3, err
    assert np.array_equal(got, ref)


def test_config0_single_layer_end_to_end():
    x = synth.activations(16, 256, seed=synth.seed_for(0, 0, synth.ROLE_ACT))
    _end_to_end(x, quantized_layer(256, 256, 0), label="C0 M=16 N=K=256")


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_config1_gemv_sweep_full_size(m):
    x = synth.activations(m, 4096, seed=synth.seed_for(1, m, synth.ROLE_ACT))
    _end_to_end(x, quantized_layer(4096, 4096, 1), label=f"C1 M={m}")


def test_config2_gemm_full_size_sampled_rows():
    x = synth.activations(2048, 4096, seed=synth.seed_for(2, 0, synth.ROLE_ACT), kind="outliers",
                          outlier_seed=synth.seed_for(2, 0, synth.ROLE_OUTLIER))
    rows = np.sort(synth.rng(22).choice(2048, 192, replace=False))
    _end_to_end(x, quantized_layer(4096, 4096, 2), rows=rows, label="C2 M=2048")


@pytest.mark.parametrize("which", ["up", "down"])
def test_config3_mlp_pair_full_size_sampled_rows(which):
    n, k = (12288, 3072) if which == "up" else (3072, 12288)
    x = synth.activations(4096, k, seed=synth.seed_for(3, 0 if which == "up" else 1, synth.ROLE_ACT),
                          kind="student_t")
    rows = np.sort(synth.rng(33).choice(4096, 96, replace=False))
    _end_to_end(x, quantized_layer(n, k, 3, 0 if which == "up" else 1), rows=rows, label=f"C3 {which}")


@pytest.mark.parametrize("n,k", [(3072, 3072), (9216, 3072), (12288, 3072), (3072, 12288)])
def test_config4_layer_shapes_decode_and_prefill(n, k):
    # one layer of each shape of the 64-layer batch, at M = 1 (GEMV) and M = 8192 (GEMM, sampled rows);
    # storage bytes drawn at random in the range a Gaussian layer's quantiser produces
    packed, srel, sch = random_layer(n, k, seed=synth.seed_for(4, n // 1024, synth.ROLE_BYTES), lo=0x58, hi=0x72)
    layer_np = (packed, srel, sch, O.FIXED_CODEBOOK)
    x1 = synth.activations(1, k, seed=synth.seed_for(4, n, synth.ROLE_ACT))
    _end_to_end(x1, layer_np, label=f"C4 M=1 {n}x{k}")
    x = synth.activations(8192, k, seed=synth.seed_for(4, n + 1, synth.ROLE_ACT))
    rows = np.sort(synth.rng(44).choice(8192, 48, replace=False))
    _end_to_end(x, layer_np, rows=rows, label=f"C4 M=8192 {n}x{k}")


def test_streams_are_respected():
    # the binding launches on the current stream; results on a side stream match
    packed, srel, sch, cb = quantized_layer(256, 256, 0)
    layer = host_layer(packed, srel, sch, cb)
    x = synth.activations(40, 256, seed=5)
    ref, *_ = O.linear(x, packed, srel, sch, cb, out="bf16")
    s = torch.cuda.Stream()
    xd = bf16_dev(x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = B.linear(xd, layer)
    s.synchronize()
    assert np.array_equal(bf16_bits(y), ref)


def test_accumulator_extremes_at_the_largest_k():
    # K = 131072, every activation +127 or -127 and every weight -128 (uniform codebook
    # code 0 = -8 at scale 16): |acc| = 127 * 128 * 131072 = 2 130 706 432, the largest the
    # ABI allows, just inside int32; the raw accumulator must be exact on both paths
    k, n = 131072, 24
    packed = np.zeros((n, k // 2), np.uint8)             # code 0 in both nibbles
    srel = np.full((n, k // 16), 0x58, np.uint8)         # e4m3 0x58 = 16.0
    sch = np.full(n, 1e-6, np.float32)
    cb = O.uniform_codebook()
    layer = host_layer(packed, srel, sch, cb)
    for m, fn in [(3, B.w4a8_gemv), (9, B.w4a8_gemm)]:
        xq_np = np.full((m, k), 127, np.int8)
        xq_np[1] = -127
        xq = torch.from_numpy(xq_np).to(DEV)
        xs = torch.ones(m, dtype=torch.float32, device=DEV)
        say("accumulator extremes", fn.__name__, m, n, k)
        got = fn(xq, xs, layer, torch.int32).cpu().numpy().astype(np.int64)
        ref = O.gemm_exact(xq_np, O.decode_w4(packed, srel, cb))
        assert ref.min() == -127 * 128 * k and ref.max() == 127 * 128 * k
        assert np.array_equal(got, ref)
