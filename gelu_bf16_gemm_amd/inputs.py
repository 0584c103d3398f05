"""Seeded synthetic inputs, shared bit for bit by the HIP path and the oracle.

This module only draws random numbers and rounds them once to the storage
type (bf16, fp16 or fp32). It holds none of the arithmetic of the fused
linear layer or the LayerNorm+GELU row kernel, so the oracle and the HIP path
can both consume its arrays without sharing any method code.

Every tensor gets its own numpy PCG64 stream ``default_rng([seed, config_id,
tensor_id])``. Distributions follow the workload descriptions: ``N(0, 1/K)``
for weights is read as a *variance* of 1/K (fan-in scaling); decimal spreads
such as 0.02 and 0.1 are read as *standard deviations*.
"""

from __future__ import annotations

import numpy as np

# Storage type codes (the same integers as the C header's dtype enum).
F32, BF16, F16, F8E4M3 = 0, 1, 2, 3

_NP_STORE = {F32: np.float32, BF16: np.uint16, F16: np.float16, F8E4M3: np.uint8}


def rng_for(config_id: int, tensor_id: int, seed: int = 0) -> np.random.Generator:
    """One independent PCG64 stream per (config, tensor)."""
    return np.random.default_rng([seed, config_id, tensor_id])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite random draws, so NaN handling is not needed here.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # u + 0x7FFF + lsb stays below 2**32 for every finite float32 bit pattern
    r = u >> 16
    r &= 1
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def store(a32: np.ndarray, dtype: int) -> np.ndarray:
    """Round a float32 array once to its storage type (bit pattern array for bf16)."""
    if dtype == F32:
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(a32)
    if dtype == F16:
        return np.ascontiguousarray(a32, dtype=np.float32).astype(np.float16)
    raise ValueError(f"unsupported storage dtype {dtype}")


def to_f64(stored: np.ndarray, dtype: int) -> np.ndarray:
    """Exact stored values as float64 (bf16 patterns decoded)."""
    if dtype == BF16:
        return bf16_bits_to_f32(stored).astype(np.float64)
    return np.asarray(stored).astype(np.float64)


def normal(rng: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    if mean != 0.0:
        z += np.float32(mean)
    return z


# ---------------------------------------------------------------------------
# Workloads. Each entry lists shapes, storage types and the distribution recipe;
# ``make_inputs`` draws them. ``config_id`` keys the random streams.
# ---------------------------------------------------------------------------

WORKLOADS = {
    # Linear + bias + GELU(erf), fp32 in/out.
    "linear_gelu_f32_64x256x256": dict(config_id=1, kind="linear", M=64, N=256, K=256,
                                       in_dtype=F32, bias=True, act="gelu_erf", out_dtype=F32),
    # LayerNorm + GELU(tanh) rows, fp16 in/out, fp32 statistics.
    "ln_gelu_f16_32768x4096": dict(config_id=2, kind="ln", rows=32768, cols=4096,
                                   io_dtype=F16, eps=1e-5, form="tanh"),
    "ln_gelu_f16_32768x3000": dict(config_id=3, kind="ln", rows=32768, cols=3000,
                                   io_dtype=F16, eps=1e-5, form="tanh"),
    # Fused QKV projection + bias, split into three 4096x4096 outputs.
    "qkv_bias_split_bf16_4096x12288x4096": dict(config_id=4, kind="linear", M=4096, N=12288, K=4096,
                                                in_dtype=BF16, bias=True, act=None, split=3,
                                                out_dtype=BF16),
    # MLP-up + bias + GELU(erf).
    "mlp_up_gelu_bf16_8192x16384x4096": dict(config_id=5, kind="linear", M=8192, N=16384, K=4096,
                                             in_dtype=BF16, bias=True, act="gelu_erf",
                                             out_dtype=BF16),
    # Out-projection + residual + store residual stream + sum-sq partials + gamma; then finalize.
    "outproj_residual_rms_bf16_16384x2048x2048": dict(config_id=6, kind="linear", M=16384, N=2048,
                                                      K=2048, in_dtype=BF16, bias=False, act=None,
                                                      residual=True, store_aux=True, rowsumsq=True,
                                                      col_scale=True, out_dtype=BF16, eps=1e-6),
    # Gate/up (pair-interleaved rows) + SwiGLU.
    "gateup_swiglu_bf16_16384x16384x2048": dict(config_id=7, kind="linear", M=16384, N=16384, K=2048,
                                                in_dtype=BF16, bias=False, act="swiglu",
                                                out_dtype=BF16),
    # Decode-shaped gate/up + SwiGLU + per-row FP8 e4m3 quantised writeback.
    "decode_swiglu_fp8_bf16_32x16384x2048": dict(config_id=8, kind="linear", M=32, N=16384, K=2048,
                                                 in_dtype=BF16, bias=False, act="swiglu",
                                                 quant_fp8=True, out_dtype=F8E4M3),
    # Same epilogue at prefill size.
    "prefill_swiglu_fp8_bf16_16384x16384x2048": dict(config_id=9, kind="linear", M=16384, N=16384,
                                                     K=2048, in_dtype=BF16, bias=False, act="swiglu",
                                                     quant_fp8=True, out_dtype=F8E4M3),
    # Pattern A end to end: the out-projection of config 6 (residual, h1, partials, gamma -> h2)
    # feeding the gate/up layer of config 7, whose epilogue applies the deferred RMSNorm row scale
    # computed from the partials (ROW_RMS) before SwiGLU.
    "chain_outproj_gateup_rms_bf16_16384x2048x16384": dict(config_id=13, kind="chain", M=16384, d=2048,
                                                           K0=2048, N2=16384, eps=1e-6, act="swiglu"),
    # LM head with the cross-entropy epilogue (32K vocabulary, hidden 2048); logits not stored.
    "lmhead_xent_bf16_4096x32768x2048": dict(config_id=14, kind="linear", M=4096, N=32768, K=2048,
                                             in_dtype=BF16, bias=False, act=None, xent=True,
                                             out_dtype=BF16),
    # The fused QKV projection with RoPE on its Q and K blocks (head width 128).
    "qkv_bias_rope_split_bf16_4096x12288x4096": dict(config_id=12, kind="linear", M=4096, N=12288,
                                                     K=4096, in_dtype=BF16, bias=True, act=None,
                                                     split=3, rope=128, out_dtype=BF16),
    # E4M3 inputs with per-row activation and per-channel weight scales: the down-projection
    # that consumes the quantised SwiGLU output above, with its residual add.
    "downproj_residual_fp8in_16384x2048x8192": dict(config_id=10, kind="linear", M=16384, N=2048,
                                                    K=8192, in_dtype=F8E4M3, bias=False, act=None,
                                                    residual=True, dequant=True, out_dtype=BF16),
    # The MLP-up layer of config 5 with E4M3 inputs (bias bf16).
    "mlp_up_gelu_fp8in_8192x16384x4096": dict(config_id=11, kind="linear", M=8192, N=16384, K=4096,
                                              in_dtype=F8E4M3, bias=True, act="gelu_erf",
                                              dequant=True, out_dtype=BF16),
}

# tensor ids inside one config
_T_X, _T_W, _T_B, _T_Z, _T_GAMMA, _T_BETA, _T_SA, _T_SW, _T_ROPE, _T_W1, _T_LAB = 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10


def random_e4m3_codes(rng: np.random.Generator, shape, e_lo: int = 4, e_hi: int = 10) -> np.ndarray:
    """Random OCP E4M3 bit patterns: uniform sign, exponent field uniform in [e_lo, e_hi], uniform
    3-bit mantissa (magnitudes 2^(e_lo-7) .. 1.875 * 2^(e_hi-7); never NaN)."""
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    exp = rng.integers(e_lo, e_hi + 1, size=shape, dtype=np.uint8) << 3
    man = rng.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign | exp | man).astype(np.uint8)


def make_linear_inputs(spec: dict, seed: int = 0, M: int | None = None, N: int | None = None,
                       K: int | None = None) -> dict:
    """Draw X (M,K), W (N,K), optional b (N), z (M,N), gamma (N) for a linear workload.

    Shapes may be overridden to get reduced cases with the same recipe.
    X ~ N(0,1); W ~ N(0, var 1/K); b ~ N(0, std 0.02); z ~ N(0,1); gamma = 1 + N(0, std 0.1).
    """
    cid = spec["config_id"]
    M = spec["M"] if M is None else M
    N = spec["N"] if N is None else N
    K = spec["K"] if K is None else K
    dt = spec["in_dtype"]
    out = {"M": M, "N": N, "K": K, "in_dtype": dt}
    vec_dt = dt if dt == F32 else BF16  # bias, residual and gamma of 16-bit and E4M3 layers are bf16
    if dt == F8E4M3:
        # codes of magnitude 1/8 .. 15 with scales around 1/8 (activations) and 1/(8 sqrt K)
        # (weights): dequantised X is O(1) and W about N(0, 1/K) in size
        out["X"] = random_e4m3_codes(rng_for(cid, _T_X, seed), (M, K))
        out["W"] = random_e4m3_codes(rng_for(cid, _T_W, seed), (N, K))
        out["sa"] = (rng_for(cid, _T_SA, seed).uniform(0.5, 1.5, size=M) / 8.0).astype(np.float32)
        out["sw"] = (rng_for(cid, _T_SW, seed).uniform(0.5, 1.5, size=N) / (8.0 * np.sqrt(K))).astype(np.float32)
    else:
        out["X"] = store(normal(rng_for(cid, _T_X, seed), (M, K)), dt)
        out["W"] = store(normal(rng_for(cid, _T_W, seed), (N, K), std=float(1.0 / np.sqrt(K))), dt)
    if spec.get("bias"):
        out["b"] = store(normal(rng_for(cid, _T_B, seed), (N,), std=0.02), vec_dt)
    if spec.get("residual"):
        out["z"] = store(normal(rng_for(cid, _T_Z, seed), (M, N)), vec_dt)
    if spec.get("col_scale"):
        out["gamma"] = store(normal(rng_for(cid, _T_GAMMA, seed), (N,), mean=1.0, std=0.1), vec_dt)
    if spec.get("xent"):
        out["labels"] = rng_for(cid, _T_LAB, seed).integers(0, N, size=M).astype(np.int32)
    if spec.get("rope"):
        # per-row cos / sin of uniformly drawn angles (a rotation table; no frequency schedule)
        d = spec["rope"]
        ang = rng_for(cid, _T_ROPE, seed).uniform(0.0, 2.0 * np.pi, size=(M, d // 2))
        cs = np.empty((M, d), np.float32)
        cs[:, 0::2], cs[:, 1::2] = np.cos(ang), np.sin(ang)
        out["rope_cs"] = cs
    return out


def make_chain_inputs(spec: dict, seed: int = 0) -> dict:
    """X (M, K0) ~ N(0,1); W0 (d, K0) var 1/K0; z (M, d) ~ N(0,1); gamma = 1 + N(0, std 0.1);
    W1 (N2, d) var 1/d; all bf16."""
    cid, M, d, K0, N2 = spec["config_id"], spec["M"], spec["d"], spec["K0"], spec["N2"]
    return {
        "X": store(normal(rng_for(cid, _T_X, seed), (M, K0)), BF16),
        "W0": store(normal(rng_for(cid, _T_W, seed), (d, K0), std=float(1.0 / np.sqrt(K0))), BF16),
        "z": store(normal(rng_for(cid, _T_Z, seed), (M, d)), BF16),
        "gamma": store(normal(rng_for(cid, _T_GAMMA, seed), (d,), mean=1.0, std=0.1), BF16),
        "W1": store(normal(rng_for(cid, _T_W1, seed), (N2, d), std=float(1.0 / np.sqrt(d))), BF16),
    }


def make_ln_inputs(spec: dict, seed: int = 0, rows: int | None = None, cols: int | None = None) -> dict:
    """Draw x (rows, cols) ~ N(0,1), gamma = 1 + N(0, std 0.1), beta ~ N(0, std 0.1), all fp16."""
    cid = spec["config_id"]
    rows = spec["rows"] if rows is None else rows
    cols = spec["cols"] if cols is None else cols
    dt = spec["io_dtype"]
    return {
        "rows": rows, "cols": cols, "io_dtype": dt,
        "x": store(normal(rng_for(cid, _T_X, seed), (rows, cols)), dt),
        "gamma": store(normal(rng_for(cid, _T_GAMMA, seed), (cols,), mean=1.0, std=0.1), dt),
        "beta": store(normal(rng_for(cid, _T_BETA, seed), (cols,), std=0.1), dt),
    }


def random_stored(rng: np.random.Generator, shape, dtype: int, mean=0.0, std=1.0) -> np.ndarray:
    """Free-form helper for tests: normal draws rounded to a storage type."""
    return store(normal(rng, shape, mean=mean, std=std), dtype)
