"""Pins for the fp64 oracle: each test checks it against something other than itself.

Pins used: brute force in pure Python on tiny shapes, worked examples with
identity / permutation / one-hot weights, closed forms (textbook normal-CDF
values, odd-part identities, asymptotics), invariants (LayerNorm moments,
RMSNorm scale invariance), split-statistics merge identities on random splits,
the exhaustive E4M3 code table, and torch's CPU float8 cast on in-range values.
No test here needs a GPU.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# brute force helpers (pure Python loops, tiny shapes only)
# ---------------------------------------------------------------------------

def bf_contract(x, w):
    M, K = len(x), len(x[0])
    N = len(w)
    out = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += x[m][k] * w[n][k]
            out[m][n] = s
    return out


def bf_gelu_erf(v):
    # 1 + erf(x) = erfc(-x): no cancellation in the negative tail
    return 0.5 * v * math.erfc(-v / math.sqrt(2.0))


def bf_gelu_tanh(v):
    c = math.sqrt(2.0 / math.pi)
    u = c * (v + 0.044715 * v ** 3)
    if u >= 0.0:
        return 0.5 * v * (1.0 + math.tanh(u))
    # u < 0: 1 + tanh u = 2 e^(2u) / (1 + e^(2u)), which does not cancel as 1 + tanh u does
    e = math.exp(2.0 * u)
    return v * e / (1.0 + e)


def bf_silu(g):
    return g / (1.0 + math.exp(-g))


# ---------------------------------------------------------------------------
# contraction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 7), (3, 2, 17), (7, 17, 3), (17, 7, 2)])
def test_contraction_brute_force_exact_integers(M, N, K):
    rng = np.random.default_rng([11, M, N, K])
    x = rng.integers(-8, 9, size=(M, K)).astype(np.float64)
    w = rng.integers(-8, 9, size=(N, K)).astype(np.float64)
    ref = np.array(bf_contract(x.tolist(), w.tolist()))
    got = O.contract(x, w)
    assert got.shape == (M, N)
    assert np.array_equal(got, ref)  # small integers: every sum is exact


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (17, 7, 17)])
def test_contraction_brute_force_random(M, N, K):
    rng = np.random.default_rng([12, M, N, K])
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K))
    ref = np.array(bf_contract(x.tolist(), w.tolist()))
    np.testing.assert_allclose(O.contract(x, w), ref, rtol=1e-12, atol=1e-12)


def test_identity_and_permutation_weights():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((5, 8))
    assert np.array_equal(O.contract(x, np.eye(8)), x)          # W = I gives h = X exactly
    perm = rng.permutation(8)
    wp = np.eye(8)[perm]                                         # row n = e_{perm[n]}
    assert np.array_equal(O.contract(x, wp), x[:, perm])         # columns permuted
    # a non-square one-hot W picks columns of X: W row n = e_{k_n}
    ks = np.array([3, 0, 7])
    assert np.array_equal(O.contract(x, np.eye(8)[ks]), x[:, ks])


def test_zero_input_gives_activation_of_bias():
    b = np.array([-1.5, -0.25, 0.0, 0.75, 2.0])
    x = np.zeros((4, 6))
    w = np.random.default_rng(14).standard_normal((5, 6))
    out = O.linear_epilogue(x, w, bias=b, act="gelu_erf")["y"]
    for m in range(4):
        for n in range(5):
            assert out[m, n] == pytest.approx(bf_gelu_erf(b[n]), abs=1e-15)


# ---------------------------------------------------------------------------
# GELU (both forms) and SiLU
# ---------------------------------------------------------------------------

def _load_cdf(name="normal_cdf.txt"):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b = line.split()
                rows.append((float(a), float(b)))
    return rows


# ---------------------------------------------------------------------------
# low-precision inputs: scale-after-accumulate dequantisation
# ---------------------------------------------------------------------------

def _finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)  # no NaN codes


@pytest.mark.parametrize("M,N,K", [(5, 3, 9), (2, 7, 4), (1, 1, 1)])
def test_dequant_contract_brute_force(M, N, K):
    # y[m][n] = sw[n] * sa[m] * sum_k xq[m][k] wq[n][k], written out element by element; M != N
    # so an activation scale applied along the wrong axis cannot pass
    rng = np.random.default_rng([21, M, N, K])
    xq = O.e4m3_decode(_finite_codes(rng, (M, K)))
    wq = O.e4m3_decode(_finite_codes(rng, (N, K)))
    sa = rng.uniform(0.01, 2.0, size=M) * rng.choice([-1.0, 1.0], size=M)
    sw = rng.uniform(0.01, 2.0, size=N)
    ref = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += xq[m, k] * wq[n, k]
            ref[m, n] = sw[n] * sa[m] * acc
    np.testing.assert_allclose(O.dequant_contract(xq, wq, sa, sw), ref, rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(O.dequant_contract(xq, wq), O.contract(xq, wq), rtol=0, atol=0)


def test_dequant_equals_dequantising_the_inputs_first():
    # one scale group over all of K: scaling after the accumulation equals contracting the
    # dequantised operands xq * sa[m] and wq * sw[n] (linearity)
    rng = np.random.default_rng(22)
    M, N, K = 6, 4, 33
    xq = O.e4m3_decode(_finite_codes(rng, (M, K)))
    wq = O.e4m3_decode(_finite_codes(rng, (N, K)))
    sa = rng.uniform(0.001, 1.0, size=M)
    sw = rng.uniform(0.001, 1.0, size=N)
    direct = O.contract(xq * sa[:, None], wq * sw[:, None])
    np.testing.assert_allclose(O.dequant_contract(xq, wq, sa, sw), direct, rtol=1e-12, atol=1e-12)


def test_dequant_integer_codes_and_power_of_two_scales_exact():
    # codes whose values are small integers and power-of-two scales: every result is exact
    ints = np.array([-4.0, -3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0, 4.0])
    codes = O.e4m3_encode(ints)
    assert np.array_equal(O.e4m3_decode(codes), ints)
    rng = np.random.default_rng(23)
    xi = rng.integers(0, len(ints), size=(4, 16))
    wi = rng.integers(0, len(ints), size=(3, 16))
    xq, wq = O.e4m3_decode(codes[xi]), O.e4m3_decode(codes[wi])
    sa = np.array([0.5, 2.0, 0.25, 8.0])
    sw = np.array([4.0, 0.125, 1.0])
    want = (ints[xi] @ ints[wi].T) * sa[:, None] * sw[None, :]
    assert np.array_equal(O.dequant_contract(xq, wq, sa, sw), want)


def test_fp8_input_worked_example_bias_is_not_scaled():
    # x codes 0x38, 0x40 (1, 2); w codes 0x38, 0x38 (1, 1); sa = 0.5, sw = 2, b = 0.25:
    # y = 0.5 * 2 * (1 + 2) + 0.25 = 3.25 (scaling the bias too would give 3.5)
    xq = O.e4m3_decode(np.array([[0x38, 0x40]], dtype=np.uint8))
    wq = O.e4m3_decode(np.array([[0x38, 0x38]], dtype=np.uint8))
    out = O.linear_epilogue(xq, wq, bias=[0.25], x_scale=[0.5], w_scale=[2.0])
    assert out["y"][0, 0] == 3.25
    out = O.linear_epilogue(xq, wq, bias=[0.25], x_scale=[0.5], w_scale=[2.0], act="gelu_erf")
    assert out["y"][0, 0] == pytest.approx(3.25 * 0.5 * (1.0 + math.erf(3.25 / math.sqrt(2.0))), rel=1e-15)


# ---------------------------------------------------------------------------
# RoPE pairwise epilogue
# ---------------------------------------------------------------------------

def test_rope_worked_examples():
    # (1, 0) by 30 degrees -> (cos 30, sin 30); (a, b) by a quarter turn (cos 0, sin 1) -> (-b, a)
    c30, s30 = math.sqrt(3.0) / 2.0, 0.5
    out = O.rope_pairs(np.array([[1.0, 0.0, 3.0, -2.0]]), np.array([[c30, s30, 0.0, 1.0]]), d=4)
    assert np.allclose(out, [[c30, s30, 2.0, 3.0]], rtol=0, atol=1e-15)
    assert out[0, 2] == 2.0 and out[0, 3] == 3.0  # exact for the quarter turn


def test_rope_inverse_norm_and_head_periodicity():
    rng = np.random.default_rng(31)
    M, d, heads = 5, 8, 3
    y = rng.standard_normal((M, d * heads))
    ang = rng.uniform(0, 2 * np.pi, size=(M, d // 2))
    cs = np.empty((M, d))
    cs[:, 0::2], cs[:, 1::2] = np.cos(ang), np.sin(ang)
    inv = cs.copy()
    inv[:, 1::2] *= -1.0
    r = O.rope_pairs(y, cs, d)
    np.testing.assert_allclose(O.rope_pairs(r, inv, d), y, rtol=0, atol=1e-12)   # rotate back
    np.testing.assert_allclose(r[:, 0::2] ** 2 + r[:, 1::2] ** 2, y[:, 0::2] ** 2 + y[:, 1::2] ** 2,
                               rtol=1e-12)                                          # pair norms kept
    # every head of d columns uses the same d/2 angles
    for h in range(heads):
        np.testing.assert_allclose(r[:, h * d:(h + 1) * d], O.rope_pairs(y[:, h * d:(h + 1) * d], cs, d),
                                   rtol=0, atol=0)


def test_rope_leaves_unrotated_columns_and_v_block():
    rng = np.random.default_rng(32)
    y = rng.standard_normal((3, 12))
    cs = O.rope_table([0, 5, 9], 4)
    r = O.rope_pairs(y, cs, 4, rot_cols=8)  # Q, K of width 4 rotated, V (last 4) untouched
    assert np.array_equal(r[:, 8:], y[:, 8:])
    assert np.array_equal(O.rope_pairs(y, O.rope_table([0, 0, 0], 4), 4), y)  # position 0: identity


def test_rope_scores_depend_on_position_difference_only():
    # the defining property of rotary embeddings: q(p) . k(p') after rotation depends on p - p'
    rng = np.random.default_rng(33)
    d = 16
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, d))
    def score(p, pp):
        qr = O.rope_pairs(q, O.rope_table([p], d), d)
        kr = O.rope_pairs(k, O.rope_table([pp], d), d)
        return float((qr * kr).sum())
    assert score(7, 3) == pytest.approx(score(104, 100), rel=1e-9, abs=1e-9)
    assert score(0, 0) == pytest.approx(float((q * k).sum()), rel=1e-12)
    assert abs(score(7, 3) - score(7, 4)) > 1e-6


# ---------------------------------------------------------------------------
# pattern A: the deferred row scale
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", [None, "swiglu"])
def test_pattern_a_equals_normalising_before_the_second_gemm(act):
    # (r h1 gamma) W1 = r (h1 gamma) W1 row by row: the deferred form equals RMSNorm first
    rng = np.random.default_rng(41)
    M, K0, N1, N2 = 6, 9, 260, 10
    x, w0 = rng.standard_normal((M, K0)), rng.standard_normal((N1, K0))
    z, gamma = rng.standard_normal((M, N1)), 1.0 + 0.1 * rng.standard_normal(N1)
    w1 = rng.standard_normal((N2, N1))
    out = O.pattern_a_chain(x, w0, z, gamma, w1, 1e-6, act=act)
    h1 = x @ w0.T + z
    normed = h1 / np.sqrt((h1 * h1).mean(axis=1, keepdims=True) + 1e-6) * gamma[None, :]
    direct = normed @ w1.T
    if act == "swiglu":
        direct = direct[:, 0::2] / (1.0 + np.exp(-direct[:, 0::2])) * direct[:, 1::2]
    np.testing.assert_allclose(out["y"], direct, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(out["r"], 1.0 / np.sqrt((h1 * h1).mean(axis=1) + 1e-6), rtol=1e-12)


# ---------------------------------------------------------------------------
# cross-entropy epilogue
# ---------------------------------------------------------------------------

def test_cross_entropy_closed_forms():
    N = 37
    assert np.allclose(O.cross_entropy(np.zeros((2, N)), [0, 36]), math.log(N), rtol=0, atol=1e-14)  # uniform
    h = np.zeros((1, N))
    h[0, 5] = 60.0
    # the exact loss 36 e^-60 ~ 3e-25 is below the fp64 resolution of lse ~ 60 (about 1e-14)
    assert O.cross_entropy(h, [5])[0] == pytest.approx((N - 1) * math.exp(-60.0), abs=1e-13)
    assert O.cross_entropy(h, [4])[0] == pytest.approx(60.0, rel=1e-12)
    assert O.cross_entropy(h, [-100])[0] == 0.0 and O.cross_entropy(h, [N])[0] == 0.0   # ignored rows
    # two classes: -log sigmoid of the margin
    assert O.cross_entropy(np.array([[1.5, -0.5]]), [0])[0] == pytest.approx(math.log1p(math.exp(-2.0)), rel=1e-14)


def test_cross_entropy_brute_force_and_shift_invariance():
    rng = np.random.default_rng(51)
    h = rng.standard_normal((4, 9)) * 3
    lab = [0, 8, 3, 5]
    want = [-h[i, lab[i]] + math.log(sum(math.exp(v) for v in h[i])) for i in range(4)]
    np.testing.assert_allclose(O.cross_entropy(h, lab), want, rtol=1e-13)
    np.testing.assert_allclose(O.cross_entropy(h + 700.0, lab), want, rtol=1e-11)   # no overflow


@pytest.mark.parametrize("N,chunk", [(1000, 128), (128, 128), (300, 64), (5, 128)])
def test_xent_chunk_stats_merge_to_the_direct_loss(N, chunk):
    rng = np.random.default_rng([52, N, chunk])
    M = 6
    h = rng.standard_normal((M, N)) * 4
    lab = rng.integers(-1, N, size=M)
    m, s = O.xent_chunk_stats(h, chunk)
    assert m.shape == (M, -(-N // chunk))
    assert np.all(s >= 1.0)            # the chunk maximum contributes e^0 = 1
    tgt = h[np.arange(M), np.clip(lab, 0, N - 1)]
    np.testing.assert_allclose(O.xent_merge_loss(m, s, tgt, lab, N), O.cross_entropy(h, lab), rtol=1e-12, atol=1e-12)


def test_gelu_erf_textbook_normal_cdf():
    for x, phi in _load_cdf():
        assert O.gelu_erf(np.array([x]))[0] == pytest.approx(x * phi, rel=1e-15, abs=1e-16)
        # GELU(-x) = -x (1 - Phi(x))
        assert O.gelu_erf(np.array([-x]))[0] == pytest.approx(-x * (1 - phi), rel=1e-13, abs=1e-16)
    assert O.gelu_erf(np.array([1.0]))[0] == pytest.approx(0.8413447460685429, rel=1e-15)
    assert O.gelu_erf(np.array([-1.0]))[0] == pytest.approx(-0.15865525393145707, rel=1e-14)


def test_gelu_erf_negative_tail_textbook():
    # GELU_erf(-x) = -x Q(x) with Q the textbook upper tail of the normal distribution: the
    # oracle keeps full relative accuracy down to GELU(-8) ~ -5e-15
    for x, q in _load_cdf("normal_tail.txt"):
        assert O.gelu_erf(np.array([-x]))[0] == pytest.approx(-x * q, rel=1e-12)
        assert bf_gelu_erf(-x) == pytest.approx(-x * q, rel=1e-12)
    # the tanh form in the same range against the scalar route through math.exp
    x = np.linspace(-12.0, -3.0, 91)
    np.testing.assert_allclose(O.gelu_tanh(x), [bf_gelu_tanh(v) for v in x], rtol=1e-12, atol=0)
    assert (O.gelu_erf(x) < 0).all() and (O.gelu_tanh(x) < 0).all()


@pytest.mark.parametrize("f", [O.gelu_erf, O.gelu_tanh])
def test_gelu_closed_forms(f):
    assert f(np.array([0.0]))[0] == 0.0
    assert f(np.array([10.0]))[0] == pytest.approx(10.0, abs=1e-20)
    assert abs(f(np.array([-10.0]))[0]) < 1e-20
    x = np.random.default_rng(15).uniform(-6, 6, 2001)
    # the odd part of GELU is x/2: GELU(x) - GELU(-x) = x for both forms
    np.testing.assert_allclose(f(x) - f(-x), x, rtol=0, atol=1e-14)
    # GELU(x) >= min value ~ -0.17 and GELU(x) <= max(x, 0)
    assert (f(x) <= np.maximum(x, 0) + 1e-15).all()
    assert (f(x) > -0.1701).all()


def test_gelu_tanh_matches_sigmoid_identity_and_page_constants():
    consts = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    x = np.linspace(-7, 7, 1401)
    # 0.5 (1 + tanh z) = 1 / (1 + e^{-2z}): an independent evaluation route
    z = math.sqrt(2 / math.pi) * (x + consts["tanh_cubic"] * x ** 3)
    np.testing.assert_allclose(O.gelu_tanh(x), x / (1 + np.exp(-2 * z)), rtol=1e-13, atol=1e-15)
    # the pages print rounded constants; they equal the exact ones in fp32
    assert np.float32(consts["erf_scale_printed"]) == np.float32(1 / math.sqrt(2))
    assert np.float32(consts["tanh_scale_printed"]) == np.float32(math.sqrt(2 / math.pi))
    # the pages put the erf/tanh gap at the 1e-3 level; the exact maximum is below it
    gap = np.abs(O.gelu_erf(x) - O.gelu_tanh(x))
    assert consts["gelu_forms_gap_magnitude"] * 0.1 < gap.max() < consts["gelu_forms_gap_magnitude"]
    assert abs(abs(x[np.argmax(gap)]) - 2.70) < 0.05


def test_gelu_scalar_brute_force():
    x = np.random.default_rng(16).normal(0, 3, 257)
    np.testing.assert_allclose(O.gelu_erf(x), [bf_gelu_erf(v) for v in x], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(O.gelu_tanh(x), [bf_gelu_tanh(v) for v in x], rtol=1e-13, atol=1e-15)


def test_silu_closed_forms():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([1.0]))[0] == pytest.approx(0.7310585786300049, rel=1e-15)  # 1/(1+1/e)
    assert O.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15
    x = np.random.default_rng(17).uniform(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(x) - O.silu(-x), x, atol=1e-12)
    assert O.silu(np.array([-1000.0]))[0] == 0.0  # no overflow to NaN


# ---------------------------------------------------------------------------
# SwiGLU pairs and the full epilogue chain against a scalar brute force
# ---------------------------------------------------------------------------

def test_swiglu_interleaved_identity_example():
    # W_gu rows 2j and 2j+1 both e_j: gate = up = x_j, so y_j = silu(x_j) * x_j
    K = 6
    w = np.zeros((2 * K, K))
    for j in range(K):
        w[2 * j, j] = 1.0
        w[2 * j + 1, j] = 1.0
    x = np.random.default_rng(18).standard_normal((4, K))
    y = O.linear_epilogue(x, w, act="swiglu")["y"]
    np.testing.assert_array_equal(y, O.silu(x) * x)
    # gate rows zero: silu(0) = 0 so every output is 0
    w2 = w.copy()
    w2[0::2] = 0.0
    assert np.array_equal(O.linear_epilogue(x, w2, act="swiglu")["y"], np.zeros((4, K)))
    # gate = e_j, up = 2 e_j -> y = 2 silu(x) x ; swapping roles must differ
    w3 = w.copy()
    w3[1::2] *= 2.0
    np.testing.assert_allclose(O.linear_epilogue(x, w3, act="swiglu")["y"], 2 * O.silu(x) * x, rtol=1e-15)
    w4 = w.copy()
    w4[0::2] *= 2.0
    assert not np.allclose(O.linear_epilogue(x, w4, act="swiglu")["y"], 2 * O.silu(x) * x)


@pytest.mark.parametrize("act", [None, "gelu_erf", "gelu_tanh", "swiglu"])
def test_epilogue_chain_brute_force(act):
    M, N, K = 5, 10, 7
    rng = np.random.default_rng([19, [None, "gelu_erf", "gelu_tanh", "swiglu"].index(act)])
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K))
    b = rng.standard_normal(N)
    z = rng.standard_normal((M, N))
    g = 1 + 0.1 * rng.standard_normal(N)
    r = rng.uniform(0.5, 1.5, M)
    got = O.linear_epilogue(x, w, bias=b, residual=z, col_scale=g, row_scale=r, act=act,
                            partial_cols=4)
    h = bf_contract(x.tolist(), w.tolist())
    h1 = [[h[m][n] + b[n] + z[m][n] for n in range(N)] for m in range(M)]
    v = [[h1[m][n] * g[n] * r[m] for n in range(N)] for m in range(M)]
    if act is None:
        y = v
    elif act == "gelu_erf":
        y = [[bf_gelu_erf(t) for t in row] for row in v]
    elif act == "gelu_tanh":
        y = [[bf_gelu_tanh(t) for t in row] for row in v]
    else:
        y = [[bf_silu(row[2 * j]) * row[2 * j + 1] for j in range(N // 2)] for row in v]
    parts = [[sum(h1[m][n] ** 2 for n in range(c, min(c + 4, N))) for c in range(0, N, 4)]
             for m in range(M)]
    np.testing.assert_allclose(got["h1"], h1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(got["y"], y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["partials"], parts, rtol=1e-12, atol=1e-13)
    assert got["partials"].shape == (M, 3)  # ragged last chunk of 2 columns


def test_residual_store_aux_and_col_scale_worked_examples():
    rng = np.random.default_rng(20)
    x = rng.standard_normal((3, 4))
    z = rng.standard_normal((3, 5))
    out = O.linear_epilogue(x, np.zeros((5, 4)), residual=z, col_scale=np.ones(5))
    assert np.array_equal(out["h1"], z)   # W = 0: h1 = z
    assert np.array_equal(out["y"], z)    # gamma = 1: h2 = h1


# ---------------------------------------------------------------------------
# RMSNorm partials and finalize
# ---------------------------------------------------------------------------

def test_partials_split_identity_and_integer_exactness():
    rng = np.random.default_rng(21)
    h = rng.standard_normal((6, 300))
    p = O.rowsumsq_partials(h)
    assert p.shape == (6, 3)
    np.testing.assert_allclose(p.sum(1), (h * h).sum(1), rtol=1e-13)
    # random splits merged by addition give the same row sums
    for _ in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 300), size=4, replace=False))
        parts = [(c * c).sum(1) for c in np.split(h, cuts, axis=1)]
        np.testing.assert_allclose(O.merge_sumsq(parts), (h * h).sum(1), rtol=1e-13)
    hi = rng.integers(-50, 51, size=(4, 256)).astype(np.float64)
    pi = O.rowsumsq_partials(hi)
    assert np.array_equal(pi[:, 0], (hi[:, :128] ** 2).sum(1))
    assert np.array_equal(pi[:, 1], (hi[:, 128:] ** 2).sum(1))


def test_finalize_closed_forms():
    eps = 1e-6
    # worked example: row (3, 4): mean square 12.5
    p = O.rowsumsq_partials(np.array([[3.0, 4.0]]))
    assert O.rmsnorm_finalize(p, 2, eps)[0] == pytest.approx(1 / math.sqrt(12.5 + eps), rel=1e-15)
    # constant row c: r = 1/sqrt(c^2 + eps)
    c = 0.37
    h = np.full((1, 2048), c)
    r = O.rmsnorm_finalize(O.rowsumsq_partials(h), 2048, eps)
    assert r[0] == pytest.approx(1 / math.sqrt(c * c + eps), rel=1e-13)
    # mean((r h)^2) = ms / (ms + eps)
    rng = np.random.default_rng(22)
    h = rng.standard_normal((8, 2048)) * rng.uniform(0.01, 3, (8, 1))
    r = O.rmsnorm_finalize(O.rowsumsq_partials(h), 2048, eps)
    ms = (h * h).mean(1)
    np.testing.assert_allclose(((r[:, None] * h) ** 2).mean(1), ms / (ms + eps), rtol=1e-12)
    # eps = 0: RMSNorm(c h) = RMSNorm(h) for c > 0
    r0 = O.rmsnorm_finalize(O.rowsumsq_partials(h), 2048, 0.0)
    r1 = O.rmsnorm_finalize(O.rowsumsq_partials(5.0 * h), 2048, 0.0)
    np.testing.assert_allclose(O.rmsnorm_apply(r0, h), O.rmsnorm_apply(r1, 5.0 * h), rtol=1e-13)


def test_rmsnorm_apply_with_gamma_brute_force():
    # y[m][n] = r[m] * h[m][n] * gamma[n], written out element by element (M != N so a
    # transposed broadcast fails), and gamma = None leaves the column factor at 1
    rng = np.random.default_rng(24)
    M, N = 3, 5
    r = rng.uniform(0.5, 2.0, M)
    h = rng.standard_normal((M, N))
    g = rng.uniform(0.5, 1.5, N)
    got = O.rmsnorm_apply(r, h, g)
    for m in range(M):
        for n in range(N):
            assert got[m, n] == pytest.approx(r[m] * h[m][n] * g[n], rel=1e-15)
    got1 = O.rmsnorm_apply(r, h)
    for m in range(M):
        for n in range(N):
            assert got1[m, n] == pytest.approx(r[m] * h[m][n], rel=1e-15)
    # worked example: row (3, 4) with eps 0 has r = 1/sqrt(12.5); gamma (2, 0.5)
    r0 = O.rmsnorm_finalize(O.rowsumsq_partials(np.array([[3.0, 4.0]])), 2, 0.0)
    y = O.rmsnorm_apply(r0, np.array([[3.0, 4.0]]), np.array([2.0, 0.5]))
    np.testing.assert_allclose(y, [[6 / math.sqrt(12.5), 2 / math.sqrt(12.5)]], rtol=1e-15)


# ---------------------------------------------------------------------------
# LayerNorm + GELU
# ---------------------------------------------------------------------------

def test_layernorm_moments_before_affine():
    rng = np.random.default_rng(23)
    x = rng.normal(3.0, 2.5, (16, 3000))
    eps = 1e-5
    xhat = O.layernorm(x, None, None, eps)
    np.testing.assert_allclose(xhat.mean(1), 0.0, atol=1e-12)
    _, var = O.layernorm_stats(x)
    np.testing.assert_allclose(xhat.var(1), var / (var + eps), rtol=1e-12)
    np.testing.assert_allclose(xhat.var(1), 1.0, atol=eps / var.min() + 1e-12)


def test_layernorm_invariances_and_constant_row():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((4, 512))
    g = 1 + 0.1 * rng.standard_normal(512)
    b = 0.1 * rng.standard_normal(512)
    base = O.layernorm(x, g, b, 0.0)
    np.testing.assert_allclose(O.layernorm(x + 7.0, g, b, 0.0), base, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(O.layernorm(3.0 * x, g, b, 0.0), base, rtol=1e-12, atol=1e-12)
    const = np.full((2, 512), 1.25)
    np.testing.assert_allclose(O.layernorm_gelu(const, g, b, 1e-5, "tanh"),
                               np.tile(O.gelu_tanh(b), (2, 1)), rtol=0, atol=1e-15)


def test_layernorm_brute_force_tiny():
    x = np.array([[1.0, 2.0, 4.0, 9.0, -3.0]])
    g = np.array([1.0, 0.5, 2.0, 1.0, -1.0])
    b = np.array([0.0, 0.1, -0.2, 0.3, 0.0])
    eps = 1e-5
    mu = sum(x[0]) / 5
    var = sum((v - mu) ** 2 for v in x[0]) / 5
    ref = [bf_gelu_tanh((x[0][i] - mu) / math.sqrt(var + eps) * g[i] + b[i]) for i in range(5)]
    np.testing.assert_allclose(O.layernorm_gelu(x, g, b, eps, "tanh")[0], ref, rtol=1e-14)


# ---------------------------------------------------------------------------
# split row statistics: merges equal direct computation on random splits
# ---------------------------------------------------------------------------

def test_chan_merge_equals_two_pass_statistics():
    rng = np.random.default_rng(25)
    for trial in range(20):
        row = rng.normal(rng.uniform(-5, 5), rng.uniform(0.1, 4), rng.integers(2, 600))
        cuts = np.sort(rng.choice(np.arange(1, len(row)), size=min(5, len(row) - 1), replace=False))
        acc = None
        for c in np.split(row, cuts):
            st = (len(c), c.mean(), ((c - c.mean()) ** 2).sum())
            acc = st if acc is None else O.merge_mean_m2(acc, st)
        mu, var = O.layernorm_stats(row[None, :])
        assert acc[0] == len(row)
        assert acc[1] == pytest.approx(mu[0], rel=1e-12, abs=1e-12)
        assert acc[2] / acc[0] == pytest.approx(var[0], rel=1e-11)


def test_online_softmax_rescale_merge_equals_direct():
    rng = np.random.default_rng(26)
    for trial in range(20):
        row = rng.normal(0, rng.uniform(0.5, 30), rng.integers(2, 500))
        cuts = np.sort(rng.choice(np.arange(1, len(row)), size=min(6, len(row) - 1), replace=False))
        st = None
        for c in np.split(row, cuts):
            loc = (c.max(), np.exp(c - c.max()).sum())
            st = loc if st is None else O.merge_max_sumexp(st, loc)
        m_direct = row.max()
        s_direct = np.exp(row - m_direct).sum()
        assert st[0] == m_direct
        assert st[1] == pytest.approx(s_direct, rel=1e-12)
        # streaming one element at a time (the m_k, d_k recurrence) agrees as well
        m, d = -np.inf, 0.0
        for v in row:
            m, d = O.merge_max_sumexp((m, d), (v, 1.0))
        assert d == pytest.approx(s_direct, rel=1e-12)


def test_max_of_maxima_equals_global_absmax():
    rng = np.random.default_rng(27)
    y = rng.standard_normal((7, 1000))
    parts = [np.abs(c).max(1) for c in np.split(y, [100, 228, 512, 900], axis=1)]
    assert np.array_equal(O.merge_absmax(parts), np.abs(y).max(1))


# ---------------------------------------------------------------------------
# E4M3 encoder and per-row quantisation
# ---------------------------------------------------------------------------

def test_e4m3_table_spot_values():
    v = O.e4m3_values()
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x08] == 2.0 ** -6          # smallest normal
    assert v[0x01] == 2.0 ** -9          # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert v[0x38] == 1.0                # exponent field 7 = bias
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    finite = v[~np.isnan(v)]
    assert len(finite) == 254


def test_e4m3_roundtrip_midpoints_and_saturation():
    v = O.e4m3_values()
    codes = np.array([c for c in range(256) if not np.isnan(v[c])], dtype=np.uint8)
    back = O.e4m3_encode(v[codes])
    assert np.array_equal(back, codes)  # every finite code round-trips (incl. -0 -> 0x80)
    pos = v[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    enc = O.e4m3_encode(mids)
    assert (enc % 2 == 0).all()          # ties go to the even code
    assert (np.abs(enc.astype(int) - np.arange(126)) <= 1).all()
    assert np.array_equal(O.e4m3_encode(-mids), enc | 0x80)
    assert len(mids) + len(mids) == 252
    # just off the midpoints rounds to the nearer neighbour
    up = O.e4m3_encode(mids * (1 + 1e-9))
    assert np.array_equal(up, np.arange(1, 127))
    assert O.e4m3_encode(np.array([464.0]))[0] == 0x7E
    assert O.e4m3_encode(np.array([1e9]))[0] == 0x7E
    assert O.e4m3_encode(np.array([-1e9]))[0] == 0xFE
    assert O.e4m3_encode(np.array([2.0 ** -6]))[0] == 0x08
    assert O.e4m3_encode(np.array([2.0 ** -9]))[0] == 0x01
    assert O.e4m3_encode(np.array([2.0 ** -11]))[0] == 0x00   # below half the smallest subnormal
    assert O.e4m3_encode(np.array([3 * 2.0 ** -11]))[0] == 0x01


def test_e4m3_ordinal_is_the_value_line():
    # Exhaustive over the 254 finite codes: sorting the codes by value, the ordinal rises with
    # the value (strictly, except that +0 and -0 share ordinal 0) and value-adjacent codes are
    # exactly one ordinal apart, so |ordinal difference| counts E4M3 steps (ulps) between codes.
    v = O.e4m3_values()
    codes = np.array([c for c in range(256) if not np.isnan(v[c])], dtype=np.uint8)
    assert len(codes) == 254
    ordn = O.e4m3_ordinal(codes)
    assert O.e4m3_ordinal(np.array([0x00]))[0] == 0 and O.e4m3_ordinal(np.array([0x80]))[0] == 0
    order = np.argsort(v[codes], kind="stable")
    vals, ords = v[codes][order], ordn[order]
    for i in range(len(vals) - 1):
        if vals[i] == vals[i + 1]:          # the two zeros
            assert vals[i] == 0.0 and ords[i] == ords[i + 1] == 0
        else:
            assert ords[i + 1] - ords[i] == 1, (vals[i], vals[i + 1])
    # the ends of the line: -448 and 448 are 126 steps from zero on either side
    assert O.e4m3_ordinal(np.array([0x7E, 0xFE])).tolist() == [126, -126]
    # a distance of 1 between neighbours across zero: the smallest subnormals of either sign
    assert O.e4m3_ordinal(np.array([0x01]))[0] - O.e4m3_ordinal(np.array([0x81]))[0] == 2
    assert O.e4m3_ordinal(np.array([0x01]))[0] - O.e4m3_ordinal(np.array([0x80]))[0] == 1


def test_e4m3_matches_torch_cast_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(28)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.normal(0, 0.01, 5000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_quantize_rows_tier1_exact():
    # integer-valued rows: absmax 448 gives s = 1 and q = e4m3(y) exactly
    y = np.array([[448.0, -3.0, 2.5, 0.0, 17.0],
                  [-224.0, 112.0, 1.0, 0.5, -0.0],
                  [0.0, 0.0, 0.0, 0.0, 0.0]])
    a = np.abs(y).max(1)
    s = O.fp8_row_scale(a)
    assert s.dtype == np.float32
    assert s[0] == np.float32(1.0) and s[1] == np.float32(0.5) and s[2] == 0.0
    q = O.quantize_fp8_rows(y, s)
    assert q[0, 0] == 0x7E and q[1, 0] == 0xFE        # the absmax element hits +-448
    assert np.array_equal(q[2], np.zeros(5, np.uint8))  # a = 0 row: all zero codes
    deq = O.e4m3_decode(q) * s.astype(np.float64)[:, None]
    # 17 sits halfway between the E4M3 neighbours 16 and 18: ties go to the even code (16)
    np.testing.assert_array_equal(deq[:2], np.array([[448, -3, 2.5, 0, 16],
                                                     [-224, 112, 1, 0.5, 0]]))


def test_fp8_scale_is_correctly_rounded_fp32_division():
    rng = np.random.default_rng(29)
    a = np.abs(rng.standard_normal(100000).astype(np.float32)) * np.float32(7.3)
    s = O.fp8_row_scale(a)
    torch = pytest.importorskip("torch")
    ref = (torch.from_numpy(a) / torch.tensor(448.0, dtype=torch.float32)).numpy()
    assert np.array_equal(s, ref)
    # every non-zero row of a quantised matrix contains a +-448 code
    y = rng.standard_normal((64, 256))
    s = O.fp8_row_scale(np.abs(y).max(1))
    q = O.quantize_fp8_rows(y, s)
    assert all(((q[m] & 0x7F) == 0x7E).any() for m in range(64))


def test_qkv_split_scaled_blocks():
    rng = np.random.default_rng(30)
    A = rng.standard_normal((8, 16))
    c = rng.standard_normal(8)
    x = rng.standard_normal((5, 16))
    y = O.linear_epilogue(x, np.vstack([A, 2 * A, 4 * A]), bias=np.concatenate([c, 2 * c, 4 * c]))["y"]
    q, k, v = O.split_cols(y, 3)
    assert np.array_equal(k, 2 * q) and np.array_equal(v, 4 * q)
    assert np.array_equal(np.hstack([q, k, v]), y)
