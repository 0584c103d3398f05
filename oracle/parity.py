"""Comparison rules and row-block parity checks of GPU outputs against the fp64 oracle.

TEST INFRASTRUCTURE ONLY, like the rest of this package: used by ``tests/`` and by the
oracle leg of ``bench.py`` (which times the oracle on sampled rows and checks the GPU's rows
with the same call), never by the product path. Takes host numpy arrays only.

Tolerances (per output kind):

* bf16 / fp16:  |y - ref| <= 2e-2 + 2e-2 |ref|, element by element.
* fp32:         |y - ref| <= 1e-4 |ref| + floor + 16 FLT_MIN. "1e-4 relative" needs a floor
  where the reference crosses zero (GELU at 0), where fp32 accumulation error does not
  vanish. For GEMM outputs the floor is the fp32 accumulation bound carried to the output:
  (K + 4) 2^-24 sum_k |x_k w_k| (plus |b|, |z| for their additions) times |gamma r| times the
  activation's derivative at the pre-activation (gemm_floor). Where that derivative vanishes
  (the negative tail of GELU) the floor vanishes too and the relative bound alone applies.
  Positive outputs (row partials, RMSNorm scales, sum-exp) take no floor. Values below the
  fp32 normal range (16 FLT_MIN) carry no relative accuracy.
* fp32 outputs of E4M3 inputs: 1e-3 sum_k |x_k w_k| |sa sw| (times the activation's
  amplification) + 1e-4 |ref|: the E4M3 matrix instruction adds each block of products with
  its own internal alignment, not with exact fp32 roundings.
* E4M3 codes:   with the GPU's own row scale s, q_ref = E4M3_RNE(clamp(v_ref / s, +-448)); the
  ordinal distance between q_gpu and q_ref is at most 1 (+0 and -0 coincide).
* FP8 scales:   bit-exact s = fl32(max |y32| / 448) against the same kernel's fp32 values y32
  (tier 2), and within the accumulation bound of the oracle's fl32(max |y| / 448).
"""

from __future__ import annotations

import numpy as np

from gelu_bf16_gemm_amd import inputs as I

from . import fusedops_oracle as O

U32 = 2.0 ** -24                                   # fp32 unit roundoff
F32_TINY = 16.0 * float(np.finfo(np.float32).tiny)  # below this, fp32 keeps no relative accuracy


# ---------------------------------------------------------------------------
# comparison rules
# ---------------------------------------------------------------------------

def check_lowp(y, ref, what: str) -> None:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = np.abs(y - ref)
    bound = 2e-2 + 2e-2 * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside 2e-2+2e-2|ref|; "
                           f"worst err {err.max():.3g} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def check_f32(y, ref, what: str, floor=0.0, rel: float = 1e-4) -> None:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    bound = rel * np.abs(ref) + floor + F32_TINY
    err = np.abs(y - ref)
    bad = err > bound
    if bad.any():
        i = np.argmax(err / bound)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside {rel}|ref| + floor; worst at "
                             f"{np.unravel_index(i, err.shape)}: err {err.flat[i]:.3g} ref {ref.flat[i]:.3g}")


def _deriv(f, v):
    """Central difference of an oracle function (tolerance bookkeeping only)."""
    d = 1e-6 * np.maximum(1.0, np.abs(v))
    return (f(v + d) - f(v - d)) / (2 * d)


def gemm_floor(K: int, mag, pre, act=None, scale=1.0):
    """The fp32 error bound of a fused-linear output carried through its epilogue.

    mag:   sum_k |x_k w_k| per pre-activation element, plus |b| and |z| when they are added
    pre:   the exact pre-activation (h1 * gamma * r, the activation's input)
    scale: |gamma r| (the factors applied after the additions)
    The pre-activation error is at most (K + 4) u mag scale (K accumulations, the bias and
    residual additions, the two scalings; Higham's gamma_n bound); the activation multiplies it
    by its derivative. SwiGLU outputs take both pair members: |silu'(g) u| dg + |silu(g)| du."""
    dpre = (K + 4) * U32 * np.asarray(mag, np.float64) * np.abs(scale)
    pre = np.asarray(pre, np.float64)
    if act is None:
        return dpre
    if act == "swiglu":
        g, u = pre[:, 0::2], pre[:, 1::2]
        return np.abs(_deriv(O.silu, g) * u) * dpre[:, 0::2] + np.abs(O.silu(g)) * dpre[:, 1::2]
    f = {"gelu_erf": O.gelu_erf, "gelu_tanh": O.gelu_tanh}[act]
    return np.abs(_deriv(f, pre)) * dpre


def check_f32_e4m3_acc(y, ref, mag, what: str) -> None:
    """fp32 outputs of E4M3 inputs. The E4M3 MFMA sums each block of 64 products with its own
    internal alignment rather than exact fp32 additions (an in-bounds probe of one instruction
    measured errors up to 2.1e-4 of the block's sum of |products| on random codes, exact sums
    when the terms align), so the bound scales with mag = sum_k |x_k w_k| |sa sw| and an
    epilogue amplification of at most 2: 1e-3 * mag + 1e-4 |ref| (mag, not a tensor-wide
    floor, covers the zero crossings)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    bound = 1e-3 * mag + 1e-4 * np.abs(ref) + F32_TINY
    err = np.abs(y - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside 1e-3 mag + 1e-4 |ref|"


def check_out(y, ref, dtype: int, what: str, floor=None) -> None:
    """16-bit outputs by the 2e-2 rule; fp32 outputs by check_f32, which then needs the
    accumulation floor of the value (gemm_floor), or 0 for values bounded away from zero."""
    if dtype == I.F32:
        assert floor is not None, f"{what}: an fp32 comparison needs its floor"
        check_f32(y, ref, what, floor)
    else:
        check_lowp(y, ref, what)


def check_fp8(codes, scales, vref, what: str) -> None:
    codes = np.asarray(codes, np.uint8)
    q_ref = O.quantize_fp8_rows(vref, scales)
    d = np.abs(O.e4m3_ordinal(codes) - O.e4m3_ordinal(q_ref))
    assert (d <= 1).all(), f"{what}: {int((d > 1).sum())} codes more than 1 ulp away (max {d.max()})"


# ---------------------------------------------------------------------------
# row-block checks of whole workloads (every output of the given rows)
# ---------------------------------------------------------------------------

def decode_weights(spec: dict, inp: dict) -> np.ndarray:
    """W of a linear workload as float64 (E4M3 codes decoded)."""
    if spec["in_dtype"] == I.F8E4M3:
        return O.e4m3_decode(inp["W"])
    return I.to_f64(inp["W"], spec["in_dtype"])


def linear_rows(spec: dict, inp: dict, rows, W64=None) -> dict:
    """The oracle's outputs for `rows` of a linear workload: h1, partials, y (after RoPE when the
    workload rotates), plus the decoded X rows and the accumulation magnitude sum_k |x_k w_k|
    (+ |b| + |z|) that fp32 floors need."""
    dt = spec["in_dtype"]
    fp8 = dt == I.F8E4M3
    X = O.e4m3_decode(inp["X"][rows]) if fp8 else I.to_f64(inp["X"][rows], dt)
    W = decode_weights(spec, inp) if W64 is None else W64
    vec_dt = I.BF16 if fp8 else dt
    b = I.to_f64(inp["b"], vec_dt) if "b" in inp else None
    z = I.to_f64(inp["z"][rows], I.BF16) if "z" in inp else None
    ref = O.linear_epilogue(X, W, bias=b, residual=z,
                            col_scale=I.to_f64(inp["gamma"], I.BF16) if "gamma" in inp else None,
                            act=spec.get("act"),
                            x_scale=inp["sa"][rows].astype(np.float64) if "sa" in inp else None,
                            w_scale=inp["sw"].astype(np.float64) if "sw" in inp else None)
    if "rope_cs" in inp:
        N, d = spec["N"], spec["rope"]
        ref["y"] = O.rope_pairs(ref["y"], inp["rope_cs"][rows].astype(np.float64), d,
                                N - N // spec["split"] if spec.get("split") else N)
    ref["X"] = X
    return ref


def _mag(ref: dict, W: np.ndarray, inp: dict, rows, dt: int) -> np.ndarray:
    mag = np.abs(ref["X"]) @ np.abs(W).T
    if "sa" in inp:
        mag = mag * inp["sa"][rows].astype(np.float64)[:, None]
    if "sw" in inp:
        mag = mag * inp["sw"].astype(np.float64)[None, :]
    if "b" in inp:
        mag = mag + np.abs(I.to_f64(inp["b"], I.BF16 if dt == I.F8E4M3 else dt))[None, :]
    if "z" in inp:
        mag = mag + np.abs(I.to_f64(inp["z"][rows], I.BF16))
    return mag


def check_linear_rows(spec: dict, inp: dict, rows, out: dict, W64=None, name: str = "") -> dict:
    """Compare every output of `rows` of a linear workload with the oracle.

    `out` holds the GPU's outputs for those rows as host arrays (keys as the workload runner's
    `outputs`: y, split, aux, partials, r, scales, stats, target, loss) and, for FP8 workloads,
    optionally y32: the same kernel's fp32 values of the same op list without quantisation,
    which the tier-2 scale rule needs. Raises AssertionError on a mismatch; returns the
    worst errors seen."""
    rows = np.asarray(rows)
    W = decode_weights(spec, inp) if W64 is None else W64
    ref = linear_rows(spec, inp, rows, W)
    dt, K, N = spec["in_dtype"], spec["K"], spec["N"]
    act = spec.get("act")
    fp8_in = dt == I.F8E4M3
    stats = {}
    need_mag = spec.get("out_dtype") == I.F32 or spec.get("xent") or spec.get("quant_fp8")
    mag = _mag(ref, W, inp, rows, dt) if need_mag and not fp8_in else None
    if spec.get("quant_fp8"):
        s = np.asarray(out["scales"]).astype(np.float32)
        codes = out["y"]
        check_fp8(codes, s, ref["y"], f"{name} codes vs oracle values")
        a_ref = np.abs(ref["y"]).max(axis=1)
        # the row absmax carries the accumulation error of its elements, (K + 4) u mag through the
        # activation, plus the few-ulp error of the activation's exp / reciprocal
        da = 1e-5 * a_ref + (gemm_floor(K, mag, ref["h1"], act).max(axis=1) if mag is not None else 2e-4 * a_ref)
        s_lo = O.fp8_row_scale(np.maximum(a_ref - da, 0.0)).astype(np.float64)
        s_hi = O.fp8_row_scale(a_ref + da).astype(np.float64)
        assert ((s >= s_lo) & (s <= s_hi)).all(), f"{name}: scale outside the accumulation bound"
        assert all(((codes[i] & 0x7F) == 0x7E).any() for i in range(len(rows)) if s[i] > 0), \
            f"{name}: a row without a +-448 code"
        if "y32" in out:
            y32 = np.asarray(out["y32"], np.float64)
            check_f32(y32, ref["y"], f"{name} fp32 values", gemm_floor(K, mag, ref["h1"], act))
            s32 = O.fp8_row_scale(np.abs(y32).max(axis=1).astype(np.float32))
            assert np.array_equal(s, s32), f"{name}: scale is not fl32(absmax / 448) of the kernel's values"
            check_fp8(codes, s, y32, f"{name} codes vs own fp32 values")
        stats["scale_rel"] = float(np.max(np.abs(s - O.fp8_row_scale(a_ref)) / np.maximum(O.fp8_row_scale(a_ref), 1e-30)))
    elif spec.get("xent"):
        lab = np.asarray(inp["labels"][rows])
        T = -(-N // 64)
        dy = gemm_floor(K, mag, ref["h1"], act)
        m_ref, s_ref = O.xent_chunk_stats(ref["y"], 64)
        dchunk = np.stack([dy[:, 64 * t:64 * (t + 1)].max(1) for t in range(T)], 1)
        st = out["stats"]
        check_f32(st[:, 0::2], m_ref, f"{name} chunk max", dchunk)
        check_f32(st[:, 1::2], s_ref, f"{name} chunk sum-exp", s_ref * np.expm1(2 * dchunk))
        idx = np.arange(len(rows))
        check_f32(out["target"], ref["y"][idx, lab], f"{name} target", dy[idx, lab])
        check_f32(out["loss"], O.cross_entropy(ref["y"], lab), f"{name} loss", 4 * dy.max(1))
    elif spec.get("split"):
        d = N // spec["split"]
        for i, blk in enumerate(out["split"]):
            check_out(blk, ref["y"][:, i * d:(i + 1) * d], spec["out_dtype"], f"{name} block {i}",
                      None if mag is None else gemm_floor(K, mag[:, i * d:(i + 1) * d], ref["h1"][:, i * d:(i + 1) * d]))
    else:
        floor = None if mag is None else gemm_floor(K, mag, ref["h1"], act)
        check_out(out["y"], ref["y"], spec["out_dtype"], f"{name} Y", floor)
        stats["y_maxerr"] = float(np.max(np.abs(np.asarray(out["y"], np.float64) - ref["y"])))
    if spec.get("store_aux"):
        check_out(out["aux"], ref["h1"], I.BF16, f"{name} h1")
    if spec.get("rowsumsq"):
        check_f32(out["partials"], ref["partials"], f"{name} partials")
        check_f32(out["r"], O.rmsnorm_finalize(ref["partials"], N, spec["eps"]), f"{name} r")
    return stats


def check_chain_rows(spec: dict, inp: dict, rows, out: dict, name: str = "") -> None:
    """Pattern A rows: h1, partials, h2 against the oracle; y against the oracle's second GEMM on
    the GPU's stored h2 rows (what the second kernel actually reads)."""
    rows = np.asarray(rows)
    ref = O.pattern_a_chain(I.to_f64(inp["X"][rows], I.BF16), I.to_f64(inp["W0"], I.BF16),
                            I.to_f64(inp["z"][rows], I.BF16), I.to_f64(inp["gamma"], I.BF16),
                            I.to_f64(inp["W1"], I.BF16), spec["eps"], act=spec["act"], h2_stored=out["h2"])
    check_out(out["h1"], ref["h1"], I.BF16, f"{name} h1")
    check_f32(out["partials"], ref["partials"], f"{name} partials")
    check_out(out["h2"], ref["h2"], I.BF16, f"{name} h2")
    check_out(out["y"], ref["y"], I.BF16, f"{name} y")


def check_ln_rows(spec: dict, inp: dict, rows, got, name: str = "") -> None:
    rows = np.asarray(rows)
    dt = spec["io_dtype"]
    ref = O.layernorm_gelu(I.to_f64(inp["x"][rows], dt), I.to_f64(inp["gamma"], dt), I.to_f64(inp["beta"], dt),
                           spec["eps"], spec["form"])
    check_out(got, ref, dt, name)
