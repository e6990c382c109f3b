"""Plain, slow CPU oracle of the ConvRot W4A8 codebook linear layer (NumPy).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

Sources.  Each function cites the page and the function or section it follows:

  [AT]  ai-toolkit, ``toolkit/util/convrot_w4a8_quant.py`` (the ConvRot W4A8
        codebook backend, qtype ``convrotw4a8``): storage contract in the module
        docstring, ``FIXED_CODEBOOK``, ``W4A8_SAT``, ``_pack_codes``,
        ``_unpack_codes``, ``unpack_w4a8_eager``, ``_assign_grid``,
        ``_assign_codes``, ``grid_levels``, ``_quantize_rotated_rows``,
        ``quantize_w4a8_rotated``, the activation-quant and GEMV Triton kernels
        (their arithmetic, not their tiling) and ``dequantize_w4a8``.
  [H3]  h3-rs 0.2.0, ``src/weights.rs``: ``fn hadamard`` and
        ``fn rotate_activation`` (the ConvRot rotation the first page imports).

Precision.  The pages fix fp32 for the stored scales, the decode product, the
quantizer's divisions and the epilogue; the oracle does those steps in numpy
float32 (IEEE, round-to-nearest-even, no fused multiply-add).  Where the pages
leave the precision open the oracle takes these readings:

  * rotation: the exact block product rounded once to fp32 (fp64 where that
    is provably exact, Python integers otherwise; a block with an infinite or
    NaN input gives NaN);
  * a row of activations without a finite maximum: scale NaN, codes 0;
  * quantizer sums (ALS): fp32 products added in fp64 in k order, then fp32;
  * int32 contraction: exact (fp64 BLAS is exact for these magnitudes, checked);
  * int32 -> fp32 and fp32 -> bf16 conversions: round-to-nearest-even;
  * a NaN decode product (an fp8 NaN scale byte) decodes to 0.

Parity pins live in ``tests/test_oracle_*.py`` (closed forms, hand-worked
values in ``tests/golden/`` -- decodes, grid levels, a full quantiser trace
through both ALS passes, an epilogue whose product order is visible --,
library special cases, brute force on small tiles, exact rational checks of
the scale steps and of the rotation).  Parity unpinned: the optimality of ``FIXED_CODEBOOK`` is taken from the
page as given (its levels are not the Lloyd-Max levels of any normal law to
better than about 0.01, so it was presumably fitted to data).  The ALS passes
are pinned by their normal equation and by the group error never rising.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "FIXED_CODEBOOK", "uniform_codebook", "ALS_ITERS", "ROT_BLOCK", "GROUP",
    "ACT_QMAX", "e4m3fn_to_f32", "f32_to_e4m3fn", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "hadamard", "rotate", "rotate_to_f32", "quant_act",
    "rotate_quant_act", "pack_codes", "unpack_codes", "decode_w4",
    "assign_codes", "grid_levels", "assign_grid", "quantize_w4_rotated", "quantize_trace",
    "nearest_level_index", "round_dyadic_to_f32",
    "quantize_w4", "gemm_exact", "epilogue", "linear", "dequantize",
    "assign_grid_stochastic", "requantize_codes", "fake_quant_rotated", "dequantize_f32",
    "ste_weight_bf16", "grad_input_exact", "interleave_rows", "swiglu_interleaved", "lora_delta",
    "lora_merge_weight",
]

F32 = np.float32

# [AT] FIXED_CODEBOOK: the sixteen sorted Lloyd-Max levels for a group-normalised
# Gaussian, as printed, each converted to fp32 (round to nearest).
FIXED_CODEBOOK = np.array(
    [-0.980602, -0.794529, -0.638165, -0.500986, -0.377321, -0.263187, -0.155210, -0.050720,
     0.052541, 0.156985, 0.265284, 0.379533, 0.502636, 0.638953, 0.794876, 0.980671],
    dtype=np.float64).astype(F32)

ALS_ITERS = 2     # [AT] _ALS_ITERS: two refinement passes of the group scale
ROT_BLOCK = 256   # [AT] ConvRotW4A8Quantizer default rotation block
GROUP = 16        # [AT] ConvRotW4A8Quantizer default group size
ACT_QMAX = 127    # symmetric int8 activations (reading: act_qmax = 127)


def uniform_codebook() -> np.ndarray:
    """[AT] ConvRotW4A8Quantizer.attach_: when no codebook is given the levels
    are the signed integers code - 8."""
    return (np.arange(16, dtype=np.float64) - 8.0).astype(F32)


# ----------------------------------------------------------------------------
# number formats

def e4m3fn_to_f32(b) -> np.ndarray:
    """OCP fp8 E4M3FN byte -> fp32 (the ``torch.float8_e4m3fn`` storage the
    [AT] group scales use).  Bias 7, 3 mantissa bits, subnormals m/8 * 2^-6,
    no infinities, bytes 0x7F and 0xFF are NaN.  Exact in fp32."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = sign * mag
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return val.astype(F32)


def f32_to_e4m3fn(x) -> np.ndarray:
    """fp32 -> E4M3FN byte with round-to-nearest-even on the mantissa, keeping
    subnormals ([AT] ``_quantize_rotated_rows`` converts s_rel with
    ``.to(torch.float8_e4m3fn)``).  Magnitudes above 464 (half-way past the
    largest finite value 448) and NaN give the NaN byte, as torch does."""
    v = np.asarray(x, dtype=F32).astype(np.float64)   # exact
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.int64)
    a = np.abs(v)
    bad = np.isnan(a) | (a > 464.0)
    a = np.where(bad, 1.0, a)
    # subnormal range: a multiple of 2^-9; the quotient is exact, rint is RNE.
    # A result of 8 is the byte 0x08, the smallest normal, as it should be.
    sub_m = np.rint(a / 2.0 ** -9).astype(np.int64)
    # normal range: a = (1 + f) * 2^e with f in [0, 1); round f to eighths (RNE)
    mant, ex = np.frexp(np.maximum(a, 2.0 ** -6))      # a = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1
    m = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    normal = (e + 7) << 3 | m
    mag = np.where(a < 2.0 ** -6, sub_m, normal)
    assert np.all(bad | (mag < 0x7F)), "finite e4m3 range exceeded"
    mag = np.where(bad, 0x7F, mag)
    return (sign | mag).astype(np.uint8)


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bfloat16 bit pattern, round to nearest even (the output cast in
    [AT] ``w4a8_gemv_kernel``'s store); NaN maps to a quiet NaN."""
    u = np.asarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    isnan = np.isnan(np.asarray(x, dtype=F32))
    rounded = np.where(isnan, (u >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(F32)


# ----------------------------------------------------------------------------
# rotation  ([H3] fn hadamard, fn rotate_activation)

def hadamard(size: int = ROT_BLOCK) -> np.ndarray:
    """[H3] fn hadamard: Kronecker powers of the symmetric 4x4 regular Hadamard
    matrix (all ones except -1 on the anti-diagonal) grown until the size is
    reached (a size that is not a power of 4 is an error), divided by sqrt(size).
    Returned in fp64 (entries +-1/16 for size 256, exact)."""
    h4 = np.array([[1, 1, 1, -1], [1, 1, -1, 1], [1, -1, 1, 1], [-1, 1, 1, 1]], dtype=np.float64)
    h, n = h4, 4
    while n < size:
        h = np.kron(h, h4)
        n *= 4
    if n != size:
        raise ValueError(f"rotation size {size} is not a power of 4")
    return h / np.sqrt(size)


def rotate(x, block: int = ROT_BLOCK) -> np.ndarray:
    """[H3] fn rotate_activation: the last dimension is cut into consecutive
    blocks of ``block`` columns and each block (a row vector) is multiplied by
    the normalised Hadamard matrix.  Computed in fp64 and returned in fp64 (a
    quality reference; ``rotate_to_f32`` is the exact parity form).  The matrix
    is symmetric and its own inverse ([AT] dequantize_w4a8 relies on applying
    it twice)."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % block:
        raise ValueError(f"block {block} does not divide {x.shape}")
    h = hadamard(block)
    y = x.reshape(-1, block) @ h
    return y.reshape(x.shape)


def round_dyadic_to_f32(num: int, exp2: int) -> np.float32:
    """The fp32 value nearest to the exact number num * 2**exp2 (Python ints),
    ties to the even significand, with fp32 subnormals (multiples of 2^-149)
    and overflow to +-infinity (the IEEE rounding of an exact value)."""
    if num == 0:
        return F32(0.0)
    neg, a = num < 0, abs(num)

    def rne_shift(v: int, s: int) -> int:        # round v / 2^s to an integer, ties to even
        if s <= 0:
            return v << -s
        q, r = v >> s, v & ((1 << s) - 1)
        half = 1 << (s - 1)
        return q + 1 if (r > half or (r == half and q & 1)) else q

    top = a.bit_length() - 1 + exp2               # floor(log2 |value|)
    if top >= -126:                               # normal range: 24 significant bits
        s = a.bit_length() - 24
        q = rne_shift(a, s)
        e = exp2 + s
        if q == 1 << 24:                          # the rounding carried into a new binade
            q, e = q >> 1, e + 1
        if q.bit_length() - 1 + e > 127:
            return F32(-np.inf if neg else np.inf)
    else:                                         # subnormal range: quantum 2^-149
        q = rne_shift(a, -149 - exp2)
        e = -149
    val = float(q) * 2.0 ** e                     # exact: q < 2^25 and a power-of-two scale
    return F32(-val if neg else val)


def _f32_parts(x):
    """Each fp32 value as (integer significand m, exponent e) with x = m * 2^e
    (subnormals included, m = 0 for zeros); int64 arrays."""
    u = np.asarray(x, dtype=F32).view(np.uint32).astype(np.int64)
    ebits = (u >> 23) & 0xFF
    frac = u & 0x7FFFFF
    m = np.where(ebits > 0, frac | (1 << 23), frac)
    e = np.where(ebits > 0, ebits - 150, -149)
    m = np.where(u >> 31 == 1, -m, m)
    return m, e


def rotate_to_f32(x, block: int = ROT_BLOCK) -> np.ndarray:
    """The block product of fp32-valued inputs (bf16 activations, fp32 weights)
    with the normalised Hadamard matrix, computed exactly and rounded once to
    fp32 (reading: no intermediate rounding).  Entries are +-1/16 and the inputs
    are dyadic, so a block's products all lie on the grid 2^(L - 4), L the
    exponent of the lowest set significand bit among its non-zero inputs, and
    every partial sum is below 16 * 2^(E + 1), E the exponent of its largest
    input.  Whenever E - L <= 44 every partial sum therefore has at most 53
    significant bits and the fp64 product (any summation order) is the exact
    value, which is then rounded once; other blocks are summed with Python
    integers and rounded by round_dyadic_to_f32.  A block holding an infinite
    or NaN input has no finite product: all its outputs are NaN here."""
    x = np.asarray(x, dtype=F32)
    if x.shape[-1] % block:
        raise ValueError(f"block {block} does not divide {x.shape}")
    blocks = x.reshape(-1, block)
    with np.errstate(over="ignore", invalid="ignore"):    # overflow to inf is the IEEE rounding
        out = (blocks.astype(np.float64) @ hadamard(block)).astype(F32)
    finite = np.isfinite(blocks).all(axis=1)
    out[~finite] = np.nan
    m, e = _f32_parts(np.where(np.isfinite(blocks), blocks, F32(0.0)))
    nz = m != 0
    lsb = e + np.where(nz, np.log2(np.where(nz, np.abs(m) & -np.abs(m), 1)).astype(np.int64), 0)
    top = e + np.where(nz, np.floor(np.log2(np.where(nz, np.abs(m), 1))).astype(np.int64), 0)
    big = np.where(nz, top, -10 ** 6).max(axis=1)
    small = np.where(nz, lsb, 10 ** 6).min(axis=1)
    wide = finite & nz.any(axis=1) & (big - small > 44)
    if np.any(wide):
        signs = np.sign(hadamard(block)).astype(np.int64)   # the +-1 pattern of H * sqrt(block)
        shift = int(np.log2(np.sqrt(block)))                 # the 1/sqrt(block) = 2^-shift factor
        for b in np.nonzero(wide)[0]:
            base = int(e[b][nz[b]].min())
            ints = [int(mi) << int(ei - base) for mi, ei in zip(m[b], e[b])]
            for i in range(block):
                total = sum(int(signs[i, j]) * ints[j] for j in range(block))
                out[b, i] = round_dyadic_to_f32(total, base - shift)
    return out.reshape(x.shape)


# ----------------------------------------------------------------------------
# activation quantisation  ([AT] w4a8_act_quant_kernel)

def quant_act(v, qmax: int = ACT_QMAX):
    """[AT] w4a8_act_quant_kernel, per row of fp32 values: amax = max |v|;
    scale = amax / qmax in fp32 (1.0 for an all-zero row); q = v / scale in
    fp32, rounded half-to-even and clamped to [-qmax, qmax].  Returns
    (int8 [M, K], fp32 [M]).  A row holding an infinite or NaN value has no
    usable scale (the page leaves it undefined); reading: its scale is NaN and
    all its codes are 0, so every output of that row is NaN downstream."""
    v = np.asarray(v, dtype=F32)
    bad = ~np.isfinite(v).all(axis=1)
    v = np.where(bad[:, None], F32(0.0), v)
    amax = np.abs(v).max(axis=1)
    scale = np.where(amax > 0, amax / F32(qmax), F32(1.0)).astype(F32)
    q = np.rint((v / scale[:, None]).astype(F32))
    q = np.clip(q, -qmax, qmax)
    scale = np.where(bad, F32(np.nan), scale).astype(F32)
    return q.astype(np.int8), scale


def rotate_quant_act(x, block: int = ROT_BLOCK, qmax: int = ACT_QMAX):
    """Rotate each row (exact, one rounding to fp32) and quantise it to int8
    with one fp32 scale per row ([AT] ConvRotW4A8Quantizer.prepare_act)."""
    return quant_act(rotate_to_f32(x, block), qmax)


# ----------------------------------------------------------------------------
# storage: pack / unpack / decode  ([AT] module docstring, _pack_codes,
# _unpack_codes, unpack_w4a8_eager, W4A8_SAT)

def pack_codes(codes) -> np.ndarray:
    """[AT] _pack_codes: codes [N, K] in 0..15 -> bytes [N, K/2]; column 2j
    goes to the low nibble of byte j and column 2j+1 to the high nibble."""
    c = np.asarray(codes).astype(np.int64)
    return ((c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)).astype(np.uint8)


def unpack_codes(packed) -> np.ndarray:
    """[AT] _unpack_codes: the inverse of pack_codes."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    n, kh = b.shape
    codes = np.empty((n, 2 * kh), dtype=np.int64)
    codes[:, 0::2] = b & 0xF
    codes[:, 1::2] = (b >> 4) & 0xF
    return codes


def decode_w4(packed, srel_u8, codebook, group: int = GROUP) -> np.ndarray:
    """[AT] module docstring + unpack_w4a8_eager with W4A8_SAT: the int8 grid
    value of weight (n, k) is codebook[code] * e4m3(srel[n, k // group]) in
    fp32, rounded half-to-even and saturated to [-128, 127].  A NaN product
    (scale byte 0x7F/0xFF) decodes to 0, as a saturating float->int8
    conversion does.  Returns int8 [N, K]."""
    codes = unpack_codes(packed)
    n, k = codes.shape
    cb = np.asarray(codebook, dtype=F32)
    s = e4m3fn_to_f32(srel_u8)
    assert s.shape == (n, k // group)
    prod = cb[codes] * np.repeat(s, group, axis=1)          # fp32 product
    r = np.rint(prod)
    r = np.where(np.isnan(r), 0.0, r)
    return np.clip(r, -128, 127).astype(np.int8)


# ----------------------------------------------------------------------------
# weight quantiser  ([AT] _assign_codes, grid_levels, _assign_grid,
# _quantize_rotated_rows, quantize_w4a8_rotated)

def nearest_level_index(values, levels) -> np.ndarray:
    """The nearest-level rule of [AT] _assign_codes (against the codebook) and
    _assign_grid, deterministic branch (against a group's int8-grid levels).
    For each value, p = the number of levels strictly below it (for
    non-decreasing levels, the left insertion point of a binary search); the
    candidate indices are p - 1 and p, each clamped into the table; the one at p
    wins only if its fp32 distance |value - level| is strictly smaller, so an
    equal distance goes to the lower index.  values [..., n]; levels either [L]
    (one table for all) or [..., L] with the same leading axes.  Returns the
    chosen indices [..., n]."""
    v = np.asarray(values, dtype=F32)
    table = np.asarray(levels, dtype=F32)
    if table.ndim == 1:
        table = np.broadcast_to(table, v.shape[:-1] + table.shape)
    size = table.shape[-1]
    below = (table[..., None, :] < v[..., :, None]).sum(axis=-1)
    cand_lo = np.clip(below - 1, 0, size - 1)
    cand_hi = np.clip(below, 0, size - 1)
    dist_lo = np.abs(v - np.take_along_axis(table, cand_lo, axis=-1))
    dist_hi = np.abs(v - np.take_along_axis(table, cand_hi, axis=-1))
    return np.where(dist_hi < dist_lo, cand_hi, cand_lo)


def assign_codes(normalized, codebook) -> np.ndarray:
    """[AT] _assign_codes: the nearest codebook index of each group-normalised
    weight (nearest_level_index against the sorted codebook)."""
    return nearest_level_index(normalized, codebook)


def grid_levels(codebook, srel_u8) -> np.ndarray:
    """[AT] grid_levels: per group, the int8-grid value of each level,
    rint(codebook * e4m3(srel)) in fp32 clamped to [-127, 127].  [N, G, 16]."""
    cb = np.asarray(codebook, dtype=F32)
    s = e4m3fn_to_f32(srel_u8)
    lv = np.rint(cb[None, None, :] * s[:, :, None])
    return np.clip(lv, -127, 127).astype(F32)


def assign_grid(target, levels) -> np.ndarray:
    """[AT] _assign_grid, deterministic branch: the nearest of each group's 16
    non-decreasing grid levels.  target [N, G, g], levels [N, G, 16] -> codes
    [N, G, g]."""
    return nearest_level_index(target, levels)


def _sum_k_f64(a):
    """Sum over the last axis, adding fp32 terms in fp64 in index order, then
    rounding once to fp32 (reading of the ALS sums)."""
    acc = np.zeros(a.shape[:-1], dtype=np.float64)
    for k in range(a.shape[-1]):
        acc = acc + a[..., k].astype(np.float64)
    return acc.astype(F32)


TINY = F32(1e-8)   # [AT] the floor of every scale and denominator in the quantiser


def _group_absmax_scale(groups):
    """Step 1 of [AT] _quantize_rotated_rows: a group's first scale is its largest
    |w|, floored at 1e-8.  groups [N, G, g] -> [N, G]."""
    return np.maximum(np.abs(groups).max(axis=-1), TINY)


def _als_scale(groups, chosen):
    """One [AT] ALS pass (_ALS_ITERS of them): for the levels chosen so far, the
    least-squares group scale sum(w * level) / sum(level^2), the denominator and
    the result each floored at 1e-8.  Products in fp32, sums by _sum_k_f64, the
    quotient an fp32 division.  groups, chosen [N, G, g] -> [N, G]."""
    num = _sum_k_f64((groups * chosen).astype(F32))
    den = np.maximum(_sum_k_f64((chosen * chosen).astype(F32)), TINY)
    return np.maximum((num / den).astype(F32), TINY)


def quantize_trace(w_rot, codebook=None, group: int = GROUP) -> dict:
    """[AT] _quantize_rotated_rows applied to every row of the rotated fp32 weight
    (rows are independent), returning every intermediate by name:
      groups          the weight cut into groups of ``group`` columns, [N, G, g];
      scale0, codes0  absmax group scale, nearest codebook index of w / scale;
      scale<p>, codes<p> for p = 1 .. ALS_ITERS: the refined scale from the
                      previous codes, and the nearest indices for it;
      row_top         per row, the largest |codebook[code] * scale| (fp32 products);
      s_channel       row_top / 127 in fp32, floored at 1e-8;
      srel            e4m3 byte of scale / s_channel (fp32 quotient, RNE);
      target          w / s_channel in fp32;
      final_codes     nearest of the group's int8-grid levels (grid_levels) to
                      the target, [N, G, g];
      packed          final_codes packed two per byte."""
    w = np.asarray(w_rot, dtype=F32)
    n, k = w.shape
    cb = FIXED_CODEBOOK if codebook is None else np.asarray(codebook, dtype=F32)
    groups = w.reshape(n, k // group, group)
    out = {"groups": groups}
    scale = _group_absmax_scale(groups)
    codes = assign_codes((groups / scale[..., None]).astype(F32), cb)
    out["scale0"], out["codes0"] = scale, codes
    for p in range(1, ALS_ITERS + 1):
        scale = _als_scale(groups, cb[codes])
        codes = assign_codes((groups / scale[..., None]).astype(F32), cb)
        out[f"scale{p}"], out[f"codes{p}"] = scale, codes
    row_top = np.abs((cb[codes] * scale[..., None]).astype(F32)).max(axis=(1, 2))
    s_channel = np.maximum((row_top / F32(127.0)).astype(F32), TINY)
    srel = f32_to_e4m3fn((scale / s_channel[:, None]).astype(F32))
    target = (groups / s_channel[:, None, None]).astype(F32)
    final = assign_grid(target, grid_levels(cb, srel))
    out.update(row_top=row_top, s_channel=s_channel, srel=srel, target=target, final_codes=final,
               packed=pack_codes(final.reshape(n, k)))
    return out


def quantize_w4_rotated(w_rot, codebook=None, group: int = GROUP):
    """[AT] quantize_w4a8_rotated: K must be a multiple of 16 and of the group
    (ValueError otherwise).  Returns (packed u8 [N, K/2], srel u8 [N, K/group],
    s_channel fp32 [N], codebook fp32 [16])."""
    w_rot = np.asarray(w_rot, dtype=F32)
    k = w_rot.shape[1]
    if k % group or k % 16:
        raise ValueError(f"K={k} must be divisible by 16 and by group={group}")
    cb = FIXED_CODEBOOK if codebook is None else np.asarray(codebook, dtype=F32)
    t = quantize_trace(w_rot, cb, group)
    return t["packed"], t["srel"], t["s_channel"], cb


def quantize_w4(w, codebook=None, block: int = ROT_BLOCK, group: int = GROUP):
    """[AT] ConvRotW4A8Quantizer.quantize_: rotate the fp32 weight (exact, one
    rounding to fp32), then quantize_w4_rotated."""
    return quantize_w4_rotated(rotate_to_f32(np.asarray(w, dtype=F32), block), codebook, group)


# ----------------------------------------------------------------------------
# contraction and epilogue  ([AT] _w4a8_linear_ste_op, w4a8_gemv_kernel)

def gemm_exact(xq, w8) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * w8[n, k] exactly ([AT] the int8 x int8 ->
    int32 product of the prefill op and the GEMV's int32 multiply-accumulate).
    Computed with fp64 BLAS: every product is below 2^14 in magnitude and every
    partial sum below 2^53, so any summation order gives the exact integer.
    Returns int64 [M, N]."""
    a = np.asarray(xq, dtype=np.int8)
    b = np.asarray(w8, dtype=np.int8)
    k = a.shape[1]
    assert b.shape[1] == k and 128 * 128 * k < 2 ** 53
    acc = a.astype(np.float64) @ b.astype(np.float64).T
    return acc.astype(np.int64)


def epilogue(acc, xs, ws, bias=None, out: str = "bf16"):
    """[AT] w4a8_gemv_kernel epilogue: y = fp32(acc) * (xs[m] * ws[n]) in fp32,
    each product rounded separately, then + bias[n] in fp32 when given, then
    the cast to the output type (bf16 round to nearest even).  ``out`` is
    'bf16' (returns uint16 bit patterns), 'f32' or 'i32' (the raw int32
    accumulator, no scaling)."""
    acc = np.asarray(acc)
    if out == "i32":
        assert np.abs(acc).max(initial=0) < 2 ** 31
        return acc.astype(np.int32)
    accf = acc.astype(F32)                                  # int -> fp32, RNE
    scale = (np.asarray(xs, dtype=F32)[:, None] * np.asarray(ws, dtype=F32)[None, :]).astype(F32)
    y = (accf * scale).astype(F32)
    if bias is not None:
        y = (y + np.asarray(bias, dtype=F32)[None, :]).astype(F32)
    if out == "f32":
        return y
    if out == "bf16":
        return f32_to_bf16_bits(y)
    raise ValueError(out)


def linear(x, packed, srel_u8, s_channel, codebook, bias=None, out: str = "bf16",
           block: int = ROT_BLOCK, group: int = GROUP, qmax: int = ACT_QMAX):
    """The whole layer on bf16-valued activations x [M, K]: rotate + per-token
    quant, decode, exact contraction, epilogue.  Returns (y, xq, xs, w8)."""
    xq, xs = rotate_quant_act(x, block, qmax)
    w8 = decode_w4(packed, srel_u8, codebook, group)
    return epilogue(gemm_exact(xq, w8), xs, s_channel, bias, out), xq, xs, w8


def dequantize(packed, srel_u8, s_channel, codebook, block: int = ROT_BLOCK, group: int = GROUP):
    """[AT] dequantize_w4a8: decoded grid times the channel scale, rotated back
    to the original basis (the rotation is an involution).  fp64 [N, K]; a
    quality reference, not a parity target."""
    w8 = decode_w4(packed, srel_u8, codebook, group).astype(np.float64)
    w_rot = w8 * np.asarray(s_channel, dtype=np.float64)[:, None]
    return rotate(w_rot, block)


# ----------------------------------------------------------------------------
# training path  ([AT] _assign_grid stochastic branch, requantize_codes_,
# fake_quant_rotated_weight, _w4a8_linear_ste_backward, dequantize_w4a8)

def assign_grid_stochastic(target, levels, u) -> np.ndarray:
    """[AT] _assign_grid with stochastic=True: the bracket below each target is
    found from its left insertion point p among the 16 non-decreasing levels (the
    count of levels below it), lo = clamp(p - 1, 0, 14); the threshold
    thr = u * (lv[lo + 1] - lv[lo]) + lv[lo] (fp32, the product rounded, then the
    sum rounded); the code is lo + 1 when target > thr, else lo.  u [N, G, g] are
    the uniform draws in [0, 1) (inputs: the page draws them with rand_like)."""
    t = np.asarray(target, dtype=F32)
    lv = np.asarray(levels, dtype=F32)
    uu = np.asarray(u, dtype=F32)
    last = lv.shape[-1] - 1
    pos = (lv[:, :, None, :] < t[:, :, :, None]).sum(axis=-1)
    lo = np.clip(pos - 1, 0, last - 1)
    lv_lo = np.take_along_axis(lv, lo.reshape(lv.shape[0], lv.shape[1], -1), axis=2).reshape(t.shape)
    lv_hi = np.take_along_axis(lv, (lo + 1).reshape(lv.shape[0], lv.shape[1], -1), axis=2).reshape(t.shape)
    width = (lv_hi - lv_lo).astype(F32)
    thr = ((uu * width).astype(F32) + lv_lo).astype(F32)
    return np.clip(lo + (t > thr), 0, last)


def requantize_codes(w, srel_u8, s_channel, codebook, rotated: bool = False, u=None,
                     block: int = ROT_BLOCK, group: int = GROUP) -> np.ndarray:
    """[AT] ConvRotW4A8Quantizer.requantize_codes_: new codes for the fp32 weight
    w [N, K] on the layer's stored group scales, channel scales and codebook (the
    grid a quantisation-aware run trains against).  The weight is rotated (exact,
    rounded once to fp32) unless ``rotated``; target = w_rot / s_channel in fp32;
    codes = nearest grid level ([AT] _assign_grid), or the unbiased stochastic
    choice between the bracketing levels when the uniform draws ``u`` [N, K] are
    given.  Returns the packed codes u8 [N, K/2]."""
    w = np.asarray(w, dtype=F32)
    n, k = w.shape
    w_rot = w if rotated else rotate_to_f32(w, block)
    target = (w_rot.reshape(n, k // group, group) / np.asarray(s_channel, dtype=F32)[:, None, None]).astype(F32)
    levels = grid_levels(codebook, srel_u8)
    if u is None:
        codes = assign_grid(target, levels)
    else:
        codes = assign_grid_stochastic(target, levels, np.asarray(u, dtype=F32).reshape(target.shape))
    return pack_codes(codes.reshape(n, k))


def fake_quant_rotated(w_rot, srel_u8, s_channel, codebook, group: int = GROUP) -> np.ndarray:
    """[AT] ConvRotW4A8Quantizer.fake_quant_rotated_weight: dequant(quant(w_rot))
    on the stored scales: the nearest grid level of w_rot / s_channel (as in
    requantize_codes) times s_channel, in fp32.  Returns fp32 [N, K]."""
    w_rot = np.asarray(w_rot, dtype=F32)
    n, k = w_rot.shape
    sch = np.asarray(s_channel, dtype=F32)
    target = (w_rot.reshape(n, k // group, group) / sch[:, None, None]).astype(F32)
    levels = grid_levels(codebook, srel_u8)
    codes = assign_grid(target, levels)
    lv = np.take_along_axis(levels, codes, axis=2)
    return (lv.reshape(n, k) * sch[:, None]).astype(F32)


def dequantize_f32(packed, srel_u8, s_channel, codebook, rotate_back: bool = True,
                   block: int = ROT_BLOCK, group: int = GROUP) -> np.ndarray:
    """[AT] dequantize_w4a8 in fp32: w8 * s_channel (fp32 product), then rotated
    back to the original basis (exact block product rounded once to fp32: the
    256 terms of a block share the row scale, so the fp64 sum is exact).  With
    ``rotate_back`` false, the rotated-basis weight w8 * s_channel.  fp32 [N, K]."""
    w8 = decode_w4(packed, srel_u8, codebook, group).astype(F32)
    w_rot = (w8 * np.asarray(s_channel, dtype=F32)[:, None]).astype(F32)
    return rotate_to_f32(w_rot, block) if rotate_back else w_rot


def ste_weight_bf16(packed, srel_u8, s_channel, codebook, group: int = GROUP) -> np.ndarray:
    """[AT] _w4a8_linear_ste_backward's weight: w8 and s_channel cast to bf16
    (w8 exactly; s_channel rounded to nearest even), their product rounded to
    bf16.  Returned as fp32 values [N, K] (each one a bf16 value)."""
    w8 = decode_w4(packed, srel_u8, codebook, group).astype(F32)         # exact in bf16
    s_b = bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(s_channel, dtype=F32)))
    prod = (w8 * s_b[:, None]).astype(F32)       # exact: 8 x 8 significant bits
    return bf16_bits_to_f32(f32_to_bf16_bits(prod))


def grad_input_exact(grad, w_bf16) -> np.ndarray:
    """[AT] _w4a8_linear_ste_backward: grad [M, N] @ w [N, K], the straight-through
    gradient with respect to the layer's (rotated) input.  Exact products of the
    bf16 values summed in fp64 (the page's bf16 matmul accumulates in fp32 and
    rounds to bf16; the comparison bound allows for both).  fp64 [M, K]."""
    return np.asarray(grad, dtype=np.float64) @ np.asarray(w_bf16, dtype=np.float64)


# ----------------------------------------------------------------------------
# variants  ([H3] interleave_rows, swiglu_interleaved, QLinear::merge_loras)

def interleave_rows(t) -> np.ndarray:
    """[H3] interleave_rows: rows [a0 .. aF-1, b0 .. bF-1] -> [a0, b0, a1, b1, ...]
    (a gate/up projection's outputs paired so SwiGLU reads neighbours)."""
    t = np.asarray(t)
    n = t.shape[0]
    if n % 2:
        raise ValueError("an even number of rows is needed")
    return t.reshape((2, n // 2) + t.shape[1:]).swapaxes(0, 1).reshape(t.shape)


def swiglu_interleaved(y) -> np.ndarray:
    """[H3] swiglu_interleaved: for the last dimension laid out (g0, u0, g1, u1, ...),
    silu(g) * u with silu(g) = g / (1 + exp(-g)); fp64 here (a reference for an
    fp32 epilogue).  [..., 2F] -> [..., F]."""
    y = np.asarray(y, dtype=np.float64)
    g, u = y[..., 0::2], y[..., 1::2]
    return g / (1.0 + np.exp(-g)) * u


def lora_delta(a, b, scale) -> np.ndarray:
    """[H3] QLinear::merge_loras delta of one adapter: scale * (B @ A), B [N, r],
    A [r, K].  Reading: the products and their sum over r in fp64, in r order
    (multiply, then add; no fused multiply-add), times the scale in fp64, rounded
    once to fp32."""
    a = np.asarray(a, dtype=F32).astype(np.float64)
    b = np.asarray(b, dtype=F32).astype(np.float64)
    acc = np.zeros((b.shape[0], a.shape[1]), dtype=np.float64)
    for r in range(a.shape[0]):
        acc = acc + b[:, r:r + 1] * a[r:r + 1, :]
    return (acc * np.float64(np.float32(scale))).astype(F32)


def lora_merge_weight(packed, srel_u8, s_channel, codebook, a, b, scale,
                      block: int = ROT_BLOCK, group: int = GROUP) -> np.ndarray:
    """[H3] QLinear::merge_loras for a ConvRot layer, in this format: dequantise
    (dequantize_f32: w8 * s_channel rotated back to the plain basis), add the
    adapter's delta (lora_delta) in fp32.  The result is the plain-basis fp32
    weight that quantize_w4 (or requantize_codes) turns back into the layer."""
    w = dequantize_f32(packed, srel_u8, s_channel, codebook, True, block, group)
    return (w + lora_delta(a, b, scale)).astype(F32)
