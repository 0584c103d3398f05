"""The benchmark's algorithmic byte counts against the byte ledger of the GEMM-epilogue page.

[Epilogue] §端到端账本 counts the per-token activation traffic of out-projection -> residual ->
RMSNorm -> gate/up in bf16: about 4d elements per token once the residual add, the RMSNorm
partial sums and the column scale ride in the first GEMM's epilogue and the row scale in the
second's (and 8d unfused), and it notes that a fused SwiGLU never writes its 2 d_ff wide
pre-activation. The fixture tests/golden/byte_ledger.json holds the page's figures; these tests
check that the byte models `bench.py` divides by (workloads.ChainRun.bytes, LinearRun.bytes)
count exactly that traffic, weights and end-point activations aside. No GPU is needed: the
models are evaluated on plain attribute holders.
"""

import json
import os
from types import SimpleNamespace

import pytest

from gelu_bf16_gemm_amd import inputs as I

WL = pytest.importorskip("gelu_bf16_gemm_amd.workloads")

LEDGER = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "byte_ledger.json")))


def chain_activation_bytes_per_token(M, d, K0, N2, swiglu=True):
    """ChainRun.bytes minus the weights, gamma, the first GEMM's input X, the second GEMM's
    output y and the row partials, per token."""
    n_out = N2 // 2 if swiglu else N2
    fake = SimpleNamespace(M=M, d=d, K0=K0, N2=N2, n_out=n_out)
    total = WL.ChainRun.bytes(fake)
    T = -(-d // 128)
    weights = 2 * (d * K0 + N2 * d) + 2 * d
    ends = 2 * M * K0 + 2 * M * n_out
    partials = M * T * 4 * 2
    return (total - weights - ends - partials) / M


@pytest.mark.parametrize("d", [LEDGER["d"], 2048])
def test_chain_moves_the_pages_fused_element_count(d):
    got = chain_activation_bytes_per_token(M=4096, d=d, K0=d, N2=2 * 4 * d)
    assert got == LEDGER["fused_elements_per_token_in_d"] * d * LEDGER["elem_bytes"]
    if d == LEDGER["d"]:
        assert got == LEDGER["fused_bytes_per_token"]
        # the fusion halves the page's unfused count
        assert 2 * got == LEDGER["unfused_bytes_per_token"]


def test_swiglu_intermediate_never_counted():
    # a fused gate/up: X and W read once, only the compacted N/2 output written; the 2 d_ff
    # pre-activation (which the page prices at about 5 d_ff elements per token unfused) is absent
    M, K, d_ff = 4096, 2048, 8192
    N = 2 * d_ff
    fake = SimpleNamespace(spec={"in_dtype": I.BF16}, M=M, N=N, K=K, out_dtype=I.BF16, n_out=d_ff, b=None,
                           sa=None, sw=None, rope_cs=None, xent=None, z=None, aux=None, gamma=None,
                           partials=None, scales=None)
    assert WL.LinearRun.bytes(fake) == 2 * (M * K + N * K) + 2 * M * d_ff
    unfused_extra = LEDGER["swiglu_unfused_extra_elements_in_dff"] * LEDGER["d_ff"] * LEDGER["elem_bytes"]
    assert round(unfused_extra / 1024) == LEDGER["swiglu_unfused_extra_kib_per_token_approx"]
