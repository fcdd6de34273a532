"""Plain float64 CPU oracle for the RaBiT residual-binary hot path (2 paths, and 3 for the 3-bit variant).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Slow and obvious by
design; numpy float64 (plus ``fractions.Fraction`` for tiny exact cases).

Sources (the pages about "RaBiT: Residual-Aware Binarization Training for
Accurate and Efficient LLMs", arXiv 2602.05367):

* paper §4.1 "Binary Building Blocks" eq.  W_hat = g ⊙ B ⊙ h
* paper §4.1 "Multi-bit Approximation via Stacking" eq.  W_hat^(k) = Σ_i g_i ⊙ B_i ⊙ h_i
* paper §4.2 "The Coupled Forward Pass", steps 1-3: B_1 = sign(W_FP),
  R_1 = W_FP − W_hat_1, B_2 = sign(R_1)
* paper §1 and abstract: each successive path is derived from the residual
  error of its predecessor; App. E.1 "Weight Packing" packs 2-bit (two
  binary weights) and 3-bit (three) models
* paper §4.3 (text under eq. for preconditioning) maps g to the output side
  and h to the input side
* paper App. E.1 "Weight Packing": 32 columns per uint32, +1 -> 0, -1 -> 1
* paper §5.4: inference is additions plus element-wise scaling

Readings where the pages are silent:

* sign(v) is +1 unless v < 0 (so +0, -0 and NaN give +1; bit = 1 iff v < 0).
* Bit t of word k holds column 32k + t (LSB first); padding bits are 0.
* Initial scales ("mean |.|" of the matrix being binarised, as the workload
  statement fixes them): g[i] = fp16_rne(rowsum_i / in), h[j] =
  fp16_rne(colsum_j / out), where the sums of |M| are float64 sums in the
  canonical order defined by ``canonical_row_sums`` / ``canonical_col_sums``,
  the division is one IEEE float64 divide and the conversion to fp16 is a
  single direct round-to-nearest-even.
* R_1 is float32 with one rounding: R = fl32(W − B_1·g_1·h_1); the product
  g_1·h_1 of two fp16 values is exact in float32.
* Three paths (the 3-bit variant): the recursion continues one step,
  R_2 = fl32(R_1 − B_2·g_2·h_2), B_3 = sign(R_2), with g_3, h_3 the mean |R_2|
  (or given); the device buffer holds the third plane as path p = 2.
* GEMV/GEMM outputs are float64 here; the GPU returns float32.

Pins (tests/test_oracle_*.py): brute-force argmin on 4x8 with Fraction (B_1,
B_2), closed-form flip rule and flip statistic (B_2), Fraction means and an
independent Fraction RNE (scales, fp16/bf16 rounding), exact rational sums on
dyadic data and fsum bounds (canonical sums), word patterns that follow from
the +1 -> 0, -1 -> 1 mapping of App. E.1 "Weight Packing" (all +1, all -1,
alternating) and round trips (pack, device layout), two formulations agreeing exactly in
Fraction (GEMV), unit-vector probes, the residual-norm identity, and
closed forms for the decode glue ops.
"""
from __future__ import annotations

from fractions import Fraction
import math

import numpy as np

__all__ = [
    "TILE_ROWS", "SEG_ROWS", "TILE_COLS", "LANE_COLS",
    "f16_rne", "bf16_rne", "frac_round_to_format",
    "canonical_row_sums", "canonical_col_sums", "canonical_total", "meanabs_scales",
    "derive", "Derived",
    "pack_words", "unpack_words", "device_planes", "device_planes_to_words",
    "planes_bytes", "weff", "gemv", "gemv_additions", "gemm",
    "frac_weff", "frac_gemv", "frac_gemv_additions",
    "rmsnorm_bf16", "silu", "attention_1tok", "mlp_block", "decode_layer",
    "normwise_rel_err",
]

# ---------------------------------------------------------------------------
# Canonical summation order for the scale sums (a reading: the pages give the
# scales as learnable parameters and fix no summation order, but the fp16
# rounding of a mean can depend on it, and B_2 depends on g_1, h_1).
#
#   column sum of column j: rows are cut into tiles of TILE_ROWS = 64 rows and
#     each tile into segments of SEG_ROWS = 16 rows. A segment is summed
#     sequentially in ascending row order starting from +0.0; the 4 segment
#     sums of a tile are added left to right; tile sums are added left to
#     right.
#   row sum of row i: columns are cut into tiles of TILE_COLS = 256 columns;
#     inside a tile "lane" l (0..63) sums the columns l, l+64, l+128, l+192
#     of the tile left to right, the 64 lane values are combined by the
#     halving tree v[l] += v[l + s] for s = 32, 16, 8, 4, 2, 1 (result v[0]);
#     tile values are added left to right starting from +0.0.
#   Ragged edges are padded with +0.0, which changes no float64 sum of
#   non-negative terms.
# ---------------------------------------------------------------------------
TILE_ROWS = 64
SEG_ROWS = 16
TILE_COLS = 256
LANE_COLS = 4


def _ceil_to(n: int, m: int) -> int:
    return ((n + m - 1) // m) * m


def canonical_row_sums(a: np.ndarray) -> np.ndarray:
    """Canonical float64 sum over columns of each row of a non-negative matrix."""
    a = np.asarray(a, dtype=np.float64)
    rows, cols = a.shape
    cp = max(_ceil_to(cols, TILE_COLS), TILE_COLS)
    p = np.zeros((rows, cp), dtype=np.float64)
    p[:, :cols] = a
    t = p.reshape(rows, cp // TILE_COLS, LANE_COLS, TILE_COLS // LANE_COLS)
    v = t[:, :, 0, :].copy()                 # lane l of a tile: columns l + 64c
    for c in range(1, LANE_COLS):
        v = v + t[:, :, c, :]
    s = TILE_COLS // LANE_COLS // 2
    while s >= 1:
        v = v[..., :s] + v[..., s:2 * s]
        s //= 2
    tiles = v[..., 0]
    total = np.zeros(rows, dtype=np.float64)
    for c in range(tiles.shape[1]):
        total = total + tiles[:, c]
    return total


def canonical_col_sums(a: np.ndarray) -> np.ndarray:
    """Canonical float64 sum over rows of each column of a non-negative matrix."""
    a = np.asarray(a, dtype=np.float64)
    rows, cols = a.shape
    rp = max(_ceil_to(rows, TILE_ROWS), TILE_ROWS)
    p = np.zeros((rp, cols), dtype=np.float64)
    p[:rows] = a
    nseg = TILE_ROWS // SEG_ROWS
    q = p.reshape(rp // TILE_ROWS, nseg, SEG_ROWS, cols)
    seg = np.zeros((rp // TILE_ROWS, nseg, cols), dtype=np.float64)
    for i in range(SEG_ROWS):
        seg = seg + q[:, :, i, :]
    tile = seg[:, 0].copy()
    for s in range(1, nseg):
        tile = tile + seg[:, s]
    total = np.zeros(cols, dtype=np.float64)
    for r in range(tile.shape[0]):
        total = total + tile[r]
    return total


# ---------------------------------------------------------------------------
# Rounding to 16-bit formats
# ---------------------------------------------------------------------------
def f16_rne(v: np.ndarray) -> np.ndarray:
    """float64 -> float16 by one direct round-to-nearest-even (numpy's cast)."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16)


def bf16_rne(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 has 8 significant bits, exponent range of float32, subnormal
    quantum 2**-133, overflow to inf.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    fin = np.isfinite(v)
    out[~fin] = v[~fin]
    x = v[fin]
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)              # exponent of the quantum
    r = np.rint(np.ldexp(x, -q))             # rint: ties to even
    y = np.ldexp(r, q)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    y = np.where(np.abs(y) > bf16_max, np.copysign(np.inf, x), y)
    out[fin] = y
    return out


def frac_round_to_format(x: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction | float:
    """Exact round-to-nearest-even of a rational to a binary float format.

    mant_bits = significant bits (11 for fp16, 8 for bf16); emin = exponent of
    the smallest normal (−14 fp16, −126 bf16); emax = exponent of the largest
    binade (15 fp16, 127 bf16). Returns a Fraction, or ±inf on overflow.
    Written from the IEEE 754 definition, independently of numpy.
    """
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2**e <= a < 2**(e+1)
    q = max(e, emin) - (mant_bits - 1)          # quantum exponent
    scaled = a / (Fraction(2) ** q)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = Fraction(fl) * Fraction(2) ** q
    largest = (Fraction(2) - Fraction(2) ** (1 - mant_bits)) * Fraction(2) ** emax
    if r > largest:
        return sign * math.inf
    return sign * r


# ---------------------------------------------------------------------------
# Derivation of the two paths (paper §4.2, coupled forward pass)
# ---------------------------------------------------------------------------
def canonical_total(row_sums: np.ndarray) -> float:
    """Canonical float64 total of the (non-negative) row sums of a matrix:
    lane l (0..63) sums rows l, l+64, l+128, ... in ascending order from +0.0,
    then the 64 lane values are combined by the halving tree
    v[l] += v[l + s], s = 32, 16, 8, 4, 2, 1 (result v[0])."""
    s = np.asarray(row_sums, dtype=np.float64)
    n = s.shape[0]
    p = np.zeros(max(_ceil_to(n, 64), 64), dtype=np.float64)
    p[:n] = s
    blocks = p.reshape(-1, 64)        # block c holds rows 64c .. 64c+63, lane l = column l
    v = np.zeros(64, dtype=np.float64)
    for c in range(blocks.shape[0]):
        v = v + blocks[c]
    w = 32
    while w >= 1:
        v = v[:w] + v[w:2 * w]
        w //= 2
    return float(v[0])


def meanabs_scales(m_abs: np.ndarray, normalized: bool = False):
    """(g, h) = fp16 mean |M| per row and per column, canonical sums.

    normalized: h is divided by the global mean mu = T / (rows cols) of |M|
    (T = canonical_total of the row sums), so that g_i h_j tracks |M_ij|
    itself rather than its square: h[j] = fp16((S_col[j] / rows) / mu), each
    division one IEEE float64 division.
    """
    rows, cols = m_abs.shape
    srow = canonical_row_sums(m_abs)
    scol = canonical_col_sums(m_abs)
    g = f16_rne(srow / np.float64(cols))
    if not normalized:
        return g, f16_rne(scol / np.float64(rows))
    mu = canonical_total(srow) / (np.float64(rows) * np.float64(cols))
    with np.errstate(divide="ignore", invalid="ignore"):
        hn = (scol / np.float64(rows)) / mu if mu != 0.0 else np.zeros_like(scol)
    return g, f16_rne(hn)


class Derived:
    """Frozen artefact of one layer: sign bits and fp16 scales of each path
    (two, or three for the 3-bit variant)."""

    def __init__(self, s1, s2, g1, h1, g2, h2, r=None, s3=None, g3=None, h3=None, r2=None):
        self.s1, self.s2 = s1, s2          # bool [out][in], True = -1
        self.g1, self.h1 = g1, h1          # float16 [out], [in]
        self.g2, self.h2 = g2, h2
        self.r = r                         # float32 residual R_1 (for pins)
        self.s3, self.g3, self.h3 = s3, g3, h3   # third path, or None
        self.r2 = r2                       # float32 residual R_2 (three paths)

    @property
    def shape(self):
        return self.s1.shape

    @property
    def n_paths(self):
        return 2 if self.s3 is None else 3

    @property
    def paths(self):
        """[(s_p, g_p, h_p)] in path order."""
        ps = [(self.s1, self.g1, self.h1), (self.s2, self.g2, self.h2)]
        if self.s3 is not None:
            ps.append((self.s3, self.g3, self.h3))
        return ps


def derive(w, mode: str = "meanabs", g1=None, h1=None, g2=None, h2=None, n_paths: int = 2,
           g3=None, h3=None) -> Derived:
    """Coupled derivation of the binary cores from one shared weight.

    paper §4.2 step 1: B_1 = sign(W_FP), with path-1 scales g_1, h_1;
    step 2: R_1 = W_FP − g_1 ⊙ B_1 ⊙ h_1; step 3: B_2 = sign(R_1).
    With n_paths = 3 the same step once more (each path corrects the residual
    of its predecessor, paper §1): R_2 = R_1 − g_2 ⊙ B_2 ⊙ h_2, B_3 = sign(R_2).
    mode "meanabs": g_p, h_p are the mean |.| of the matrix being binarised
    (W for path 1, R_1 for path 2, R_2 for path 3). mode
    "meanabs_normalized": the same with h_p divided by the matrix's global
    mean |.| (``meanabs_scales``), so that g_p h_p tracks |M| (a reading
    that fits the pages' App. B Corollary 1, W_hat_2 close to R_1). mode
    "given": the scales are supplied by the caller (the last path's scales
    do not affect the bits).
    """
    if n_paths not in (2, 3):
        raise ValueError(n_paths)
    w = np.asarray(w, dtype=np.float32)
    out, inp = w.shape
    s1 = w < 0
    norm = mode == "meanabs_normalized"
    if norm:
        mode = "meanabs"
    if mode == "meanabs":
        g1, h1 = meanabs_scales(np.abs(w).astype(np.float64), norm)
    elif mode == "given":
        g1 = np.asarray(g1, dtype=np.float16)
        h1 = np.asarray(h1, dtype=np.float16)
    else:
        raise ValueError(mode)
    e1 = g1.astype(np.float32)[:, None] * h1.astype(np.float32)[None, :]
    # the fp16 x fp16 product is exact in float32
    assert np.array_equal(e1.astype(np.float64),
                          g1.astype(np.float64)[:, None] * h1.astype(np.float64)[None, :])
    b1e1 = np.where(s1, -e1, e1).astype(np.float32)
    r = (w - b1e1).astype(np.float32)          # float32 subtraction: one rounding
    s2 = r < 0
    if mode == "meanabs":
        g2, h2 = meanabs_scales(np.abs(r).astype(np.float64), norm)
    else:
        g2 = np.asarray(g2 if g2 is not None else np.zeros(out), dtype=np.float16)
        h2 = np.asarray(h2 if h2 is not None else np.zeros(inp), dtype=np.float16)
    if n_paths == 2:
        return Derived(s1, s2, g1, h1, g2, h2, r)
    # third path: the residual of path 2, with the same single float32 rounding
    e2 = g2.astype(np.float32)[:, None] * h2.astype(np.float32)[None, :]
    b2e2 = np.where(s2, -e2, e2).astype(np.float32)
    r2 = (r - b2e2).astype(np.float32)
    s3 = r2 < 0
    if mode == "meanabs":
        g3, h3 = meanabs_scales(np.abs(r2).astype(np.float64), norm)
    else:
        g3 = np.asarray(g3 if g3 is not None else np.zeros(out), dtype=np.float16)
        h3 = np.asarray(h3 if h3 is not None else np.zeros(inp), dtype=np.float16)
    return Derived(s1, s2, g1, h1, g2, h2, r, s3, g3, h3, r2)


# ---------------------------------------------------------------------------
# Packing (paper App. E.1, "Weight Packing")
# ---------------------------------------------------------------------------
def pack_words(s: np.ndarray) -> np.ndarray:
    """Canonical words: word[i][k] = Σ_t s[i, 32k+t] << t (LSB first), padding 0."""
    s = np.asarray(s, dtype=bool)
    rows, cols = s.shape
    nw = (cols + 31) // 32
    p = np.zeros((rows, nw * 32), dtype=np.uint64)
    p[:, :cols] = s
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    words = (p.reshape(rows, nw, 32) * weights).sum(axis=-1)
    return words.astype(np.uint32)


def unpack_words(words: np.ndarray, cols: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint32)
    rows, nw = words.shape
    bits = (words[:, :, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)
    return bits.reshape(rows, nw * 32)[:, :cols].astype(bool)


def planes_bytes(out: int, inp: int, n_paths: int = 2) -> int:
    """Bytes of the device plane buffer (see ``device_planes``)."""
    rg = (out + 63) // 64
    kg = (inp + 127) // 128
    return rg * kg * n_paths * 64 * 16


def device_planes(words1: np.ndarray, words2: np.ndarray, out: int, inp: int,
                  words3: np.ndarray | None = None) -> np.ndarray:
    """Device layout of the planes, written from the header's description.

    The buffer is a sequence of 16-byte units indexed (rg, kg, p, r) in
    row-major order with rg = row group of 64 rows, kg = group of 128 columns,
    p = path (0 .. n_paths − 1) and r = row inside the group (0..63). The unit
    holds, as four little-endian uint32, the canonical words 4*kg + 0..3 of row
    64*rg + r of path p. Rows >= out and words beyond the last are zero.
    Returns a flat uint32 array.
    """
    rg = (out + 63) // 64
    kg = (inp + 127) // 128
    planes = (words1, words2) if words3 is None else (words1, words2, words3)
    buf = np.zeros((rg, kg, len(planes), 64, 4), dtype=np.uint32)
    for p, words in enumerate(planes):
        rows, nw = words.shape
        for i in range(rows):
            g, r = divmod(i, 64)
            for k in range(nw):
                buf[g, k // 4, p, r, k % 4] = words[i, k]
    return buf.reshape(-1)


def device_planes_to_words(buf: np.ndarray, out: int, inp: int, n_paths: int = 2):
    """Inverse of ``device_planes`` (returns canonical words of every plane)."""
    rg = (out + 63) // 64
    kg = (inp + 127) // 128
    nw = (inp + 31) // 32
    b = np.asarray(buf, dtype=np.uint32).reshape(rg, kg, n_paths, 64, 4)
    res = []
    for p in range(n_paths):
        t = b[:, :, p].transpose(0, 2, 1, 3).reshape(rg * 64, kg * 4)
        res.append(t[:out, :nw].copy())
    return tuple(res)


# ---------------------------------------------------------------------------
# Inference linear layer (paper §4.1 eqs.; §5.4 "additions and element-wise
# scaling"; App. E.1 "per-path parallelizable")
# ---------------------------------------------------------------------------
def weff(d: Derived) -> np.ndarray:
    """W_eff = Σ_p g_p ⊙ B_p ⊙ h_p in float64 (each term exact; paths added
    in order)."""
    res = np.zeros(d.s1.shape, dtype=np.float64)
    for s, g, h in d.paths:
        res = res + g.astype(np.float64)[:, None] * np.where(s, -1.0, 1.0) * h.astype(np.float64)[None, :]
    return res


def gemv(d: Derived, x: np.ndarray) -> np.ndarray:
    """y[b, i] = Σ_j W_eff[i, j] x[b, j] in float64; x is [batch][in]."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return x @ weff(d).T


def gemv_additions(d: Derived, x: np.ndarray) -> np.ndarray:
    """Second formulation: per path, add the h-scaled inputs whose bit is +1,
    subtract those whose bit is −1, then scale by g (paper §5.4, App. E.1)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    y = np.zeros((x.shape[0], d.s1.shape[0]), dtype=np.float64)
    for s, g, h in d.paths:
        u = x * h.astype(np.float64)[None, :]
        plus = u @ (~s).astype(np.float64).T
        minus = u @ s.astype(np.float64).T
        y += g.astype(np.float64)[None, :] * (plus - minus)
    return y


def gemm(d: Derived, xm: np.ndarray, rows=None) -> np.ndarray:
    """Prefill: Y[m, n] for the token rows ``rows`` (default all)."""
    xm = np.asarray(xm, dtype=np.float64)
    if rows is not None:
        xm = xm[rows]
    return xm @ weff(d).T


def frac_weff(d: Derived):
    out, inp = d.s1.shape
    res = [[Fraction(0)] * inp for _ in range(out)]
    for s, g, h in d.paths:
        for i in range(out):
            gi = Fraction(float(g[i]))
            for j in range(inp):
                b = -1 if s[i, j] else 1
                res[i][j] += gi * b * Fraction(float(h[j]))
    return res


def frac_gemv(d: Derived, x) -> list:
    """Exact rational y = W_eff x for tiny inputs."""
    w = frac_weff(d)
    xs = [[Fraction(float(v)) for v in row] for row in np.atleast_2d(x)]
    return [[sum((wi[j] * xb[j] for j in range(len(xb))), Fraction(0)) for wi in w] for xb in xs]


def frac_gemv_additions(d: Derived, x) -> list:
    out, inp = d.s1.shape
    res = []
    for xb in np.atleast_2d(x):
        xf = [Fraction(float(v)) for v in xb]
        row = []
        for i in range(out):
            acc = Fraction(0)
            for s, g, h in d.paths:
                plus = sum((Fraction(float(h[j])) * xf[j] for j in range(inp) if not s[i, j]), Fraction(0))
                minus = sum((Fraction(float(h[j])) * xf[j] for j in range(inp) if s[i, j]), Fraction(0))
                acc += Fraction(float(g[i])) * (plus - minus)
            row.append(acc)
        res.append(row)
    return res


# ---------------------------------------------------------------------------
# Decode glue (a reading: the pages do not define a decode step; a Llama
# block is used, with plain stand-ins around the binary linear layers)
# ---------------------------------------------------------------------------
def rmsnorm_bf16(x: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """bf16(x / sqrt(mean(x^2) + eps)) per row, unit weight."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    ms = np.mean(x * x, axis=1, keepdims=True)
    return bf16_rne(x / np.sqrt(ms + eps))


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def attention_1tok(v: np.ndarray, n_heads: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """Attention over a context of one token: the softmax over a single key is
    1, so head h returns the value vector of its key/value group."""
    v = np.atleast_2d(np.asarray(v, dtype=np.float64))
    rep = n_heads // n_kv_heads
    out = np.empty((v.shape[0], n_heads * head_dim), dtype=np.float64)
    for h in range(n_heads):
        grp = h // rep
        out[:, h * head_dim:(h + 1) * head_dim] = v[:, grp * head_dim:(grp + 1) * head_dim]
    return out


def mlp_block(x_bf16: np.ndarray, gate: Derived, up: Derived, down: Derived,
              eps: float = 1e-5, norm: bool = True, residual: bool = True) -> np.ndarray:
    """x + down(bf16(silu(gate(n)) * up(n))), n = rmsnorm(x); bf16 at each
    rounding point the GPU rounds at."""
    x = np.atleast_2d(np.asarray(x_bf16, dtype=np.float64))
    n = rmsnorm_bf16(x, eps) if norm else x
    gt = gemv(gate, n)
    u = gemv(up, n)
    z = bf16_rne(silu(gt) * u)
    d = gemv(down, z)
    return bf16_rne(x + d) if residual else d


def decode_layer(x_bf16: np.ndarray, mats: dict, cfg: dict) -> np.ndarray:
    """One Llama decoder layer at a context of one token. ``mats`` maps
    q, k, v, o, gate, up, down to Derived (q..o may be absent)."""
    x = np.atleast_2d(np.asarray(x_bf16, dtype=np.float64))
    eps = cfg.get("rms_eps", 1e-5)
    if mats.get("q") is not None:
        n1 = rmsnorm_bf16(x, eps)
        # q and k are computed by the layer but do not affect a one-key softmax
        v = bf16_rne(gemv(mats["v"], n1))
        a = bf16_rne(attention_1tok(v, cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]))
        o = gemv(mats["o"], a)
        x = bf16_rne(x + o)
    return mlp_block(x, mats["gate"], mats["up"], mats["down"], eps)


def normwise_rel_err(y: np.ndarray, yref: np.ndarray) -> float:
    """max over batch rows of max_i |y − ŷ| / max_i |ŷ|."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    yref = np.atleast_2d(np.asarray(yref, dtype=np.float64))
    num = np.max(np.abs(y - yref), axis=1)
    den = np.max(np.abs(yref), axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))
