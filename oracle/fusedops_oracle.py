"""Plain, slow, fp64 definitions of everything the fused-linear library computes.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.

Pages cited (by title; section / equation / table on that page):

* [Fusion]   "Triton 算子融合: Linear+GELU、QKV 投影与注意力" (aiqz.cc,
             triton-operator-fusion-linear-attention)
* [LN+GELU]  "什么是算子融合？LayerNorm与GeLU融合如何为深度学习推理提速" (ipipp.com)
* [Softmax]  "Triton Softmax 与 FlashAttention" (aiqz.cc, triton-softmax-flash-attention)
* [Epilogue] "GEMM Epilogue 完全拆解:推理内核的最后一公里——累加器布局、融合归约与量化写回"
             (pinghaoyang.com.cn)

Each function computes the plain definition the method reaches (up to rounding
order). Every value is float64; inputs are the exact stored values (bf16 / fp16 /
fp32 decoded to float64). Nothing here rounds to bf16/fp16: the tests compare
the GPU's rounded outputs with these unrounded references under a tolerance.

Readings of the pages where they are silent or ambiguous (each is also listed
in the repository's design notes):

* W is N x K ("row n = output neuron"), so Y = X W^T.
* GELU constants: the pages print 0.70710678 and 0.7978845608; the oracle uses
  the exact 1/sqrt(2) and sqrt(2/pi) (both round to the same fp32).
* The RMSNorm aux reduction "reduce" is the mean over the N columns:
  r = 1/sqrt(sum_t p[m,t] / N + eps).
* Row partials cover fixed 128-column chunks of the pre-rounding h1.
* FP8 is OCP E4M3FN (max 448); s = fl32(absmax / 448); values are clamped to
  +-448 before round-to-nearest-even, so the encoder saturates, never NaN.
* SwiGLU reads gate = column 2j and up = column 2j+1: y_j = silu(gate) * up.
* RoPE: adjacent feature pairs (2i, 2i+1) rotate by the angle of pair index
  (column mod d) / 2 of the row's token; cos / sin come from a per-row table
  (the caller gathers it by position); with a Q/K/V split, V is not rotated.
* FP8 inputs: one scale group spanning all of K, i.e. one activation scale per
  row of X and one weight scale per row of W (output channel); both multiply the
  fp32 accumulator before the bias, which stays a 16-bit float vector.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erfc as _erfc
from scipy.special import expit as _expit

__all__ = [
    "PARTIAL_COLS", "E4M3_MAX",
    "contract", "dequant_contract", "gelu_erf", "gelu_tanh", "silu", "swiglu_pairs",
    "linear_epilogue", "rowsumsq_partials", "rmsnorm_finalize", "rmsnorm_apply",
    "layernorm_stats", "layernorm", "layernorm_gelu",
    "merge_sumsq", "merge_absmax", "merge_mean_m2", "merge_max_sumexp",
    "e4m3_values", "e4m3_decode", "e4m3_encode", "e4m3_ordinal",
    "fp8_row_scale", "quantize_fp8_rows", "split_cols", "rope_pairs", "rope_table", "pattern_a_chain",
    "cross_entropy", "xent_chunk_stats", "xent_merge_loss",
]

PARTIAL_COLS = 128          # public granularity of the RMSNorm row partials
E4M3_MAX = 448.0            # largest finite OCP E4M3FN value

_SQRT_HALF = math.sqrt(0.5)             # the Fusion page's 0.70710678
_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)  # the LN+GELU page's 0.7978845608
_GELU_CUBIC = 0.044715


# ---------------------------------------------------------------------------
# Contraction and activations
# ---------------------------------------------------------------------------

def contract(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """h[m,n] = sum_k X[m,k] W[n,k].

    [Fusion] §Linear算子剖析, equation Y_{m,n} (without the bias term), with W
    stored N x K (row n = output neuron). A float64 library matmul is the step.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ w.T


def dequant_contract(xq: np.ndarray, wq: np.ndarray, x_scale=None, w_scale=None) -> np.ndarray:
    """y[m,n] = sw[n] * sa[m] * sum_k xq[m,k] wq[n,k], the scale-after-accumulate form.

    [Epilogue] §量化尾声的完整形态, "尾声里的量化权重反解与 per-group scale": the
    accumulator keeps the unscaled partial sum over a group g of K and the epilogue
    multiplies it by the weight scale of (n, g) and the activation scale of (m, g).
    Here there is one group covering all of K. xq and wq are the decoded values of
    the stored low-precision codes (fp64); a missing scale is 1.
    """
    h = contract(xq, wq)
    if x_scale is not None:
        h = h * np.asarray(x_scale, dtype=np.float64)[:, None]
    if w_scale is not None:
        h = h * np.asarray(w_scale, dtype=np.float64)[None, :]
    return h


def gelu_erf(h: np.ndarray) -> np.ndarray:
    """GELU, erf form: 0.5 h (1 + erf(h / sqrt 2)) = h * Phi(h).

    [Fusion] §GELU激活融合 (the kernel line that applies erf to acc/sqrt 2) and
    the Python demo's epilogue. Written with 1 + erf(x) = erfc(-x), the same
    function: for h << 0 the sum 1 + erf(h / sqrt 2) cancels in float64 (at
    h = -8 it keeps about one correct digit) while erfc keeps full relative
    accuracy in the negative tail.
    """
    h = np.asarray(h, dtype=np.float64)
    return 0.5 * h * _erfc(-h * _SQRT_HALF)


def gelu_tanh(h: np.ndarray) -> np.ndarray:
    """GELU, tanh form: 0.5 h (1 + tanh(u)), u = sqrt(2/pi) (h + 0.044715 h^3).

    [Fusion] §GELU激活融合, the GELU(x) approximation equation; [LN+GELU]
    §用Triton手写融合内核 (the ``inner`` / ``gelu_out`` lines). Evaluated as
    h / (1 + e^(-2u)), the same function (1 + tanh u = 2 / (1 + e^(-2u))), so
    that the negative tail does not cancel in 1 + tanh u.
    """
    h = np.asarray(h, dtype=np.float64)
    inner = _SQRT_2_OVER_PI * (h + _GELU_CUBIC * h * h * h)
    return h * _expit(2.0 * inner)


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + e^-g) ([Epilogue] §背景, the SiLU activation)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_pairs(h: np.ndarray) -> np.ndarray:
    """Pairwise SwiGLU on adjacent feature pairs: y[:, j] = silu(h[:, 2j]) * h[:, 2j+1].

    [Epilogue] §模式B (GEMM → 逐对激活): the pair (h_a, h_b) of adjacent output
    features maps to one value, gate times value; the output width halves and is
    written compacted (§末尾布局调整).
    """
    h = np.asarray(h, dtype=np.float64)
    if h.shape[-1] % 2:
        raise ValueError("SwiGLU needs an even number of columns")
    return silu(h[..., 0::2]) * h[..., 1::2]


# ---------------------------------------------------------------------------
# Epilogue chain
# ---------------------------------------------------------------------------

def rowsumsq_partials(h1: np.ndarray, partial_cols: int = PARTIAL_COLS) -> np.ndarray:
    """p[m,t] = sum over columns n in [t*c, min((t+1)*c, N)) of h1[m,n]^2.

    [Epilogue] §六类尾声原语 item 5 (tile reduction) and §模式A "Epilogue 1"
    (the partialRMS term): per-tile row sums of squares of h1.
    """
    h1 = np.asarray(h1, dtype=np.float64)
    M, N = h1.shape
    T = -(-N // partial_cols)
    p = np.zeros((M, T), dtype=np.float64)
    for t in range(T):
        blk = h1[:, t * partial_cols:(t + 1) * partial_cols]
        p[:, t] = (blk * blk).sum(axis=1)
    return p


def linear_epilogue(x, w, bias=None, residual=None, col_scale=None, row_scale=None,
                    act=None, partial_cols: int = PARTIAL_COLS, x_scale=None, w_scale=None) -> dict:
    """The fused linear layer and its epilogue chain, in its fixed order.

    h  = sa[m] sw[n] (X W^T) + b                see dequant_contract (sa, sw only for
                                                low-precision inputs; 1 otherwise)
    h  = X W^T + b                              [Fusion] §Linear算子剖析, Y_{m,n}
    h1 = h + z                                  [Epilogue] §模式A, Epilogue 1
    p  = row sum-of-squares partials of h1      [Epilogue] §模式A, partialRMS
    h2 = h1 * gamma[n]                          [Epilogue] §模式A, Epilogue 1
    h3 = r[m] * h2                              [Epilogue] §模式A, Epilogue 2
    y  = act(h3)   act in {None, gelu_erf, gelu_tanh, swiglu}

    Returns a dict with 'h1' (the value a STORE_AUX op writes), 'partials',
    and 'y' (the main output before any rounding or quantisation).
    """
    h = dequant_contract(x, w, x_scale, w_scale)
    if bias is not None:
        h = h + np.asarray(bias, dtype=np.float64)[None, :]
    h1 = h if residual is None else h + np.asarray(residual, dtype=np.float64)
    partials = rowsumsq_partials(h1, partial_cols)
    v = h1
    if col_scale is not None:
        v = v * np.asarray(col_scale, dtype=np.float64)[None, :]
    if row_scale is not None:
        v = v * np.asarray(row_scale, dtype=np.float64)[:, None]
    if act is None:
        y = v
    elif act == "gelu_erf":
        y = gelu_erf(v)
    elif act == "gelu_tanh":
        y = gelu_tanh(v)
    elif act == "swiglu":
        y = swiglu_pairs(v)
    else:
        raise ValueError(f"unknown activation {act!r}")
    return {"h1": h1, "partials": partials, "y": y}


def rope_pairs(y: np.ndarray, cs: np.ndarray, d: int, rot_cols: int | None = None) -> np.ndarray:
    """Rotate adjacent feature pairs: (a, b) -> (a cos - b sin, a sin + b cos).

    [Epilogue] §背景 (RoPE rotates each adjacent pair of dimensions), §模式B (a pairwise map
    returning two values), §末尾布局调整 (the width is unchanged) and §用形状与步长把约定钉死 (the
    QKV output carries rotated Q and K segments, V as computed). Column pair
    (2j, 2j+1) of row m uses the angle of pair index i = (2j mod d) / 2 within its head of d
    columns: cos = cs[m, 2i], sin = cs[m, 2i+1]. Columns at or past rot_cols stay as they are.
    """
    y = np.asarray(y, dtype=np.float64)
    cs = np.asarray(cs, dtype=np.float64)
    M, N = y.shape
    rot = N if rot_cols is None else rot_cols
    out = y.copy()
    for c in range(0, rot, 2):
        i = (c % d) // 2
        cos, sin = cs[:, 2 * i], cs[:, 2 * i + 1]
        a, b = y[:, c], y[:, c + 1]
        out[:, c] = a * cos - b * sin
        out[:, c + 1] = a * sin + b * cos
    return out


def rope_table(positions, d: int, base: float = 10000.0) -> np.ndarray:
    """cos / sin of pos * base^(-2i/d) for i < d/2, interleaved per row (the usual RoPE
    frequency schedule; used by pins only, the library takes any table)."""
    pos = np.asarray(positions, dtype=np.float64)
    inv = base ** (-2.0 * np.arange(d // 2) / d)
    ang = pos[:, None] * inv[None, :]
    cs = np.empty((pos.size, d))
    cs[:, 0::2], cs[:, 1::2] = np.cos(ang), np.sin(ang)
    return cs


def split_cols(y: np.ndarray, n: int) -> list:
    """Q = H[:, :d], K = H[:, d:2d], V = H[:, 2d:] for n = 3 ([Fusion] §QKV投影融合, column slices)."""
    y = np.asarray(y)
    if y.shape[1] % n:
        raise ValueError("width not divisible by the split count")
    d = y.shape[1] // n
    return [y[:, i * d:(i + 1) * d] for i in range(n)]


def rmsnorm_finalize(partials: np.ndarray, n_cols: int, eps: float) -> np.ndarray:
    """r[m] = 1 / sqrt(sum_t p[m,t] / N + eps).

    [Epilogue] §模式A: the auxiliary kernel merges the per-tile partials by row
    and takes the root and reciprocal, r = 1/sqrt(reduce(r̂) + eps); with
    r = 1/rms(.) the reduction is read as the mean over the N columns.
    """
    p = np.asarray(partials, dtype=np.float64)
    return 1.0 / np.sqrt(p.sum(axis=1) / float(n_cols) + float(eps))


def rmsnorm_apply(r: np.ndarray, h: np.ndarray, gamma=None) -> np.ndarray:
    """y[m,n] = r[m] * h[m,n] (* gamma[n]); [Epilogue] §模式A, Epilogue 2 (row scale)."""
    y = np.asarray(r, dtype=np.float64)[:, None] * np.asarray(h, dtype=np.float64)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)[None, :]
    return y


# ---------------------------------------------------------------------------
# LayerNorm + GELU rows
# ---------------------------------------------------------------------------

def pattern_a_chain(x, w0, z, gamma, w1, eps: float, act=None, h2_stored=None) -> dict:
    """GEMM -> residual -> RMSNorm -> GEMM with the row scale deferred ([Epilogue] §模式A):

        Epilogue 1: h1 = x W0 + z,  h2 = h1 * gamma,  partials of h1 (128-column chunks)
        r = 1 / sqrt(sum_t p[m,t] / N1 + eps)           (the light aux reduction)
        Epilogue 2: y = act(r[m] * (h2 W1))

    `h2_stored`, when given, is the stored (rounded) h2 the second GEMM actually reads;
    otherwise the exact h2 is used. Returns h1, h2, partials, r and y.
    """
    e1 = linear_epilogue(x, w0, residual=z, col_scale=gamma)
    h1, h2 = e1["h1"], e1["y"]
    r = rmsnorm_finalize(e1["partials"], h1.shape[1], eps)
    x2 = h2 if h2_stored is None else np.asarray(h2_stored, dtype=np.float64)
    e2 = linear_epilogue(x2, w1, row_scale=r, act=act)
    return {"h1": h1, "h2": h2, "partials": e1["partials"], "r": r, "y": e2["y"]}


def layernorm_stats(x: np.ndarray):
    """Per-row mean and biased variance, two passes: mu = sum x / N, var = sum (x-mu)^2 / N.

    [LN+GELU] §用Triton手写融合内核: fp32 statistics in the kernel; here fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[1]
    mu = x.sum(axis=1) / n
    d = x - mu[:, None]
    var = (d * d).sum(axis=1) / n
    return mu, var


def layernorm(x: np.ndarray, gamma, beta, eps: float) -> np.ndarray:
    """(x - mu) * rstd * gamma + beta with rstd = 1/sqrt(var + eps) ([LN+GELU] §用Triton手写融合内核)."""
    x = np.asarray(x, dtype=np.float64)
    mu, var = layernorm_stats(x)
    rstd = 1.0 / np.sqrt(var + float(eps))
    xhat = (x - mu[:, None]) * rstd[:, None]
    out = xhat
    if gamma is not None:
        out = out * np.asarray(gamma, dtype=np.float64)[None, :]
    if beta is not None:
        out = out + np.asarray(beta, dtype=np.float64)[None, :]
    return out


def layernorm_gelu(x, gamma, beta, eps: float, form: str = "tanh") -> np.ndarray:
    """GELU(LayerNorm(x)) per row; form 'tanh' (the page's kernel), 'erf', or 'none'."""
    y = layernorm(x, gamma, beta, eps)
    if form == "tanh":
        return gelu_tanh(y)
    if form == "erf":
        return gelu_erf(y)
    if form == "none":
        return y
    raise ValueError(f"unknown GELU form {form!r}")


# ---------------------------------------------------------------------------
# Split row statistics: merging per-chunk statistics into whole-row ones
# ---------------------------------------------------------------------------

def merge_sumsq(parts) -> np.ndarray:
    """Sum-of-squares partials merge by addition ([Epilogue] §模式A, reduce(r̂))."""
    return np.sum(np.asarray(parts, dtype=np.float64), axis=0)


def merge_absmax(parts) -> np.ndarray:
    """Per-tile absolute maxima merge by max ([Epilogue] §仿射量化与尾声的五步, step 1)."""
    return np.max(np.asarray(parts, dtype=np.float64), axis=0)


def merge_mean_m2(a, b):
    """Merge (count, mean, M2) of two chunks (Chan et al.'s pairwise update).

    M2 is the sum of squared deviations from the chunk mean, so var = M2 / count.
    This is how a wavefront can combine per-lane LayerNorm statistics.
    """
    na, ma, m2a = a
    nb, mb, m2b = b
    n = na + nb
    delta = mb - ma
    mean = ma + delta * (nb / n)
    m2 = m2a + m2b + delta * delta * (na * nb / n)
    return n, mean, m2


def merge_max_sumexp(a, b):
    """Merge two (m, s) running statistics: m = max(m1, m2), s = s1 e^{m1-m} + s2 e^{m2-m}.

    [Softmax] §在线 Softmax (the m_k, d_k recurrence) and [Epilogue] §模式C
    (merging two segments' statistics).
    """
    m1, s1 = a
    m2, s2 = b
    m = np.maximum(m1, m2)
    return m, s1 * np.exp(m1 - m) + s2 * np.exp(m2 - m)


# ---------------------------------------------------------------------------
# Cross-entropy over the output columns (a stateful epilogue plus a final merge)
# ---------------------------------------------------------------------------

def cross_entropy(h: np.ndarray, labels) -> np.ndarray:
    """l[i] = -h[i, y_i] + log sum_k exp(h[i, k]) ([Epilogue] §模式C); rows whose label is
    outside [0, N) are ignored (loss 0). The log-sum-exp is taken around the row maximum."""
    h = np.asarray(h, dtype=np.float64)
    lab = np.asarray(labels, dtype=np.int64)
    mx = h.max(axis=1)
    lse = mx + np.log(np.exp(h - mx[:, None]).sum(axis=1))
    ok = (lab >= 0) & (lab < h.shape[1])
    tgt = np.where(ok, h[np.arange(h.shape[0]), np.clip(lab, 0, h.shape[1] - 1)], 0.0)
    return np.where(ok, lse - tgt, 0.0)


def xent_chunk_stats(h: np.ndarray, chunk: int = PARTIAL_COLS):
    """Per row and per `chunk`-column block t: m[i,t] = max_j h[i,j], s[i,t] = sum_j e^(h[i,j]-m[i,t])
    over the block's columns (the per-tile running statistics of [Epilogue] §模式C)."""
    h = np.asarray(h, dtype=np.float64)
    M, N = h.shape
    T = -(-N // chunk)
    m = np.empty((M, T))
    s = np.empty((M, T))
    for t in range(T):
        blk = h[:, t * chunk:(t + 1) * chunk]
        m[:, t] = blk.max(axis=1)
        s[:, t] = np.exp(blk - m[:, t][:, None]).sum(axis=1)
    return m, s


def xent_merge_loss(m: np.ndarray, s: np.ndarray, target, labels, n_cols: int) -> np.ndarray:
    """The final merge along the vocabulary: fold the chunks' (m, s) with merge_max_sumexp, then
    l = m + log s - target for rows with a label in [0, n_cols), 0 otherwise."""
    m = np.asarray(m, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    acc = (m[:, 0], s[:, 0])
    for t in range(1, m.shape[1]):
        acc = merge_max_sumexp(acc, (m[:, t], s[:, t]))
    lab = np.asarray(labels, dtype=np.int64)
    ok = (lab >= 0) & (lab < n_cols)
    return np.where(ok, acc[0] + np.log(acc[1]) - np.asarray(target, dtype=np.float64), 0.0)


# ---------------------------------------------------------------------------
# FP8 E4M3 (OCP E4M3FN): value table, encoder, per-row quantisation
# ---------------------------------------------------------------------------

def e4m3_values() -> np.ndarray:
    """Value of each of the 256 codes: sign bit, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; there is no
    infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_values()
_POS = _E4M3[:0x7F]          # codes 0x00..0x7E, increasing values 0 .. 448


def e4m3_decode(codes) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 value with ties to the even code, after clamping to +-448.

    [Epilogue] §仿射量化与尾声的五步, step 2: scale, round, clamp to
    [-qmax, qmax]; rounding to FP8 aligns the exponent and rounds the mantissa.
    Negative inputs keep the sign bit (so -tiny encodes as 0x80, negative zero).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no E4M3 encoding here")
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")       # _POS[hi-1] < a <= _POS[hi]
    hi = np.clip(hi, 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def e4m3_ordinal(codes) -> np.ndarray:
    """Position on the E4M3 value line (+0 and -0 share 0); used for ulp distances."""
    c = np.asarray(codes, dtype=np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def fp8_row_scale(absmax) -> np.ndarray:
    """s = fl32(a / 448): the division in float64, then one rounding to float32.

    [Epilogue] §仿射量化与尾声的五步: s = max / qmax. Because float64 holds more
    than twice float32's precision, this equals correctly rounded fp32 division
    of the float32 value a by 448.
    """
    a = np.asarray(absmax, dtype=np.float64)
    return (a / E4M3_MAX).astype(np.float32)


def quantize_fp8_rows(y, scales) -> np.ndarray:
    """q[m,j] = e4m3_RNE(clamp(y[m,j] / s[m], +-448)); a row with s = 0 is all 0x00.

    [Epilogue] §仿射量化与尾声的五步, steps 2 and 5 (values plus a per-row scale
    side-array; dequantise as q * s[m]).
    """
    y = np.asarray(y, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    out = np.zeros(y.shape, dtype=np.uint8)
    nz = s != 0.0
    if nz.any():
        t = y[nz] / s[nz][:, None]
        out[nz] = e4m3_encode(np.clip(t, -E4M3_MAX, E4M3_MAX))
    return out
