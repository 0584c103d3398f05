"""The C-ABI boundary on the CPU: the library loads, exports every symbol the header
declares, and every argument check returns its status before anything is enqueued.

Pointers here are fake, aligned addresses: each call is expected to return at a
host-side check and never touch the device (no GPU is needed or used).
"""

import ctypes
import os
import re

import pytest

from gelu_bf16_gemm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fusedops.h")

A = 0x7F0000000000  # fake 16-byte-aligned base address; regions below are spaced far apart


def addr(i: int, off: int = 0) -> int:
    return A + i * (1 << 32) + off


def test_header_symbols_are_exported():
    text = open(HEADER).read()
    decls = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fusedops_[a-z_0-9]+)\s*\(", text, re.M))
    assert decls == set(B.EXPORTS)
    for name in decls:
        assert hasattr(B.lib, name), name


def test_constants():
    assert B.abi_version() == 5
    assert B.partial_cols() == 128
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(B.status_string(s), str) and B.status_string(s)
    assert B.status_string(0) == "ok"
    text = open(HEADER).read()
    assert "#define FUSEDOPS_PARTIAL_COLS 128" in text
    assert "#define FUSEDOPS_ABI_VERSION 5" in text
    assert "#define FUSEDOPS_NOALLOC_SCRATCH_BYTES (32u << 20)" in text


def lin(X=addr(0), ldx=64, W=addr(1), ldw=64, bias=None, M=32, N=64, K=64, in_dt=B.BF16, ops=(),
        Y=addr(2), ldy=64, out_dt=B.BF16, ws=None, ws_bytes=0):
    arr, n = B.op_array(list(ops))
    return B.lib.fusedops_linear_epilogue(X, ldx, W, ldw, bias, M, N, K, in_dt, arr, n, Y, ldy, out_dt,
                                          ws, ws_bytes, None)


def mkop(kind, dtype=B.BF16, inp=None, out=None, ld=0, out_v=None, n_split=0, reserved=0):
    o = B.Op()
    o.kind, o.dtype, o.ld, o.n_split, o.reserved = kind, dtype, ld, n_split, reserved
    if inp is not None:
        o.in_ = inp
    if out is not None:
        o.out = out
    if out_v:
        for i, p in enumerate(out_v):
            o.out_v[i] = p
    return o


def test_linear_invalid_arguments():
    assert lin(X=None) == B.ERR_INVALID_ARG
    assert lin(W=None) == B.ERR_INVALID_ARG
    assert lin(Y=None) == B.ERR_INVALID_ARG
    assert lin(M=0) == B.ERR_INVALID_ARG
    assert lin(N=-8) == B.ERR_INVALID_ARG
    assert lin(K=0) == B.ERR_INVALID_ARG
    assert lin(in_dt=9) == B.ERR_INVALID_ARG
    assert lin(out_dt=-1) == B.ERR_INVALID_ARG
    assert lin(ldx=32) == B.ERR_INVALID_ARG          # ldx < K
    assert lin(ldw=56) == B.ERR_INVALID_ARG          # ldw < K
    assert lin(ldy=32) == B.ERR_INVALID_ARG          # ldy < N
    assert lin(out_dt=B.F8E4M3) == B.ERR_INVALID_ARG  # fp8 only with QUANT_FP8_ROW


def test_linear_unsupported():
    assert lin(in_dt=B.F16) == B.ERR_UNSUPPORTED
    split = mkop(B.OP_SPLIT_COLS, out_v=[addr(3), addr(4)], n_split=2, ld=16)
    assert lin(ops=[mkop(B.OP_SWIGLU), split], Y=None) == B.ERR_UNSUPPORTED


def test_fp8_input_rules():
    # every case is refused before any launch (the addresses are placeholders)
    row = mkop(B.OP_DEQUANT_ROW, dtype=B.F32, inp=addr(5))
    col = mkop(B.OP_DEQUANT_COL, dtype=B.F32, inp=addr(6))
    assert lin(in_dt=B.F8E4M3, K=8, ldx=64, ldw=64) == B.ERR_MISALIGNED        # K multiple of 16
    assert lin(in_dt=B.F8E4M3, K=64, ldx=72, ldw=64, ops=[row, col]) == B.ERR_MISALIGNED  # 72-byte rows
    assert lin(in_dt=B.BF16, ops=[row]) == B.ERR_INVALID_ARG                     # scales of FP8 inputs only
    assert lin(in_dt=B.BF16, ops=[col]) == B.ERR_INVALID_ARG
    assert lin(in_dt=B.F8E4M3, ops=[mkop(B.OP_DEQUANT_ROW, dtype=B.F32)]) == B.ERR_INVALID_ARG  # no input
    assert lin(in_dt=B.F8E4M3, ops=[col, row]) == B.ERR_INVALID_ARG              # kind order
    assert lin(in_dt=B.F8E4M3, ops=[mkop(B.OP_DEQUANT_ROW, dtype=B.F32, inp=addr(2))]) == B.ERR_INVALID_ARG  # aliases Y
    assert lin(in_dt=B.F8E4M3, ldx=32, ops=[row, col]) == B.ERR_INVALID_ARG      # ldx < K
    assert lin(in_dt=B.F8E4M3, ops=[mkop(B.OP_DEQUANT_ROW, dtype=B.F32, inp=addr(5) + 2)]) == B.ERR_MISALIGNED


def test_rope_rules():
    # every case is refused before any launch (the addresses are placeholders); N = 64
    def rope(d, ld=64, inp=addr(7), dtype=B.F32):
        o = mkop(B.OP_ROPE, dtype=dtype, inp=inp, ld=ld)
        o.n_split = d
        return o
    assert lin(ops=[rope(12)]) == B.ERR_INVALID_ARG                     # d not a multiple of 8
    assert lin(ops=[rope(0)]) == B.ERR_INVALID_ARG
    assert lin(ops=[rope(48)]) == B.ERR_INVALID_ARG                     # 64 columns not a multiple of d
    assert lin(ops=[rope(32, ld=16)]) == B.ERR_INVALID_ARG              # ld < d
    assert lin(ops=[rope(32, inp=None)]) == B.ERR_INVALID_ARG           # no table
    assert lin(ops=[rope(32, dtype=B.BF16)]) == B.ERR_INVALID_ARG       # table must be fp32
    assert lin(N=64, ldy=32, ops=[mkop(B.OP_SWIGLU), rope(32)]) == B.ERR_INVALID_ARG  # not with SwiGLU
    assert lin(ops=[rope(32, ld=34)]) == B.ERR_MISALIGNED               # 136-byte table rows
    assert lin(ops=[rope(32, inp=addr(7, 8))]) == B.ERR_MISALIGNED
    assert lin(ops=[rope(32, inp=addr(2))]) == B.ERR_INVALID_ARG        # table overlaps Y
    split = mkop(B.OP_SPLIT_COLS, out_v=[addr(3), addr(4), addr(5)], n_split=3, ld=32)
    assert lin(N=96, Y=None, ops=[split, rope(48)]) == B.ERR_INVALID_ARG  # Q+K width 64 vs d = 48


def test_row_rms_rules():
    import struct
    def rms(width=64, eps=1e-6, ld=1, inp=addr(7)):
        o = mkop(B.OP_ROW_RMS, dtype=B.F32, inp=inp, ld=ld)
        o.n_split = width
        o.reserved = int.from_bytes(struct.pack("<f", eps), "little", signed=True)
        return o
    assert lin(ops=[rms(eps=0.0)]) == B.ERR_INVALID_ARG                 # eps must be > 0
    assert lin(ops=[rms(eps=float("inf"))]) == B.ERR_INVALID_ARG
    assert lin(ops=[rms(width=0)]) == B.ERR_INVALID_ARG
    assert lin(ops=[rms(width=300, ld=2)]) == B.ERR_INVALID_ARG         # ld < ceil(300 / 128)
    assert lin(ops=[rms(inp=None)]) == B.ERR_INVALID_ARG
    assert lin(ops=[mkop(B.OP_ROW_SCALE, dtype=B.F32, inp=addr(6)), rms()]) == B.ERR_INVALID_ARG  # both scales
    assert lin(ops=[rms(inp=addr(7, 2))]) == B.ERR_MISALIGNED
    assert lin(ops=[rms(inp=addr(2))]) == B.ERR_INVALID_ARG             # partials overlap Y
    assert lin(ops=[mkop(B.OP_GELU_ERF, reserved=7)]) == B.ERR_INVALID_ARG  # reserved only for ROW_RMS


def test_xent_rules():
    def xe(labels=addr(7), stats=addr(8), target=addr(9), ld=2):
        o = mkop(B.OP_XENT, dtype=B.F32, inp=labels, out=stats, ld=ld)
        if target is not None:
            o.out_v[0] = target
        return o
    # N = 64: one 64-column chunk, so ld >= 2
    assert lin(ops=[xe(ld=1)]) == B.ERR_INVALID_ARG
    assert lin(ops=[xe(labels=None)]) == B.ERR_INVALID_ARG
    assert lin(ops=[xe(target=None)]) == B.ERR_INVALID_ARG
    assert lin(ops=[mkop(B.OP_SWIGLU), xe()], ldy=32) == B.ERR_INVALID_ARG
    assert lin(ops=[xe(stats=addr(2))]) == B.ERR_INVALID_ARG             # statistics overlap Y
    assert lin(ops=[xe(target=addr(8, 4))]) == B.ERR_INVALID_ARG        # target overlaps statistics
    assert lin(ops=[xe(labels=addr(7, 2))]) == B.ERR_MISALIGNED
    assert lin(Y=None, ops=[]) == B.ERR_INVALID_ARG                     # Y may be NULL only with XENT
    f = B.lib.fusedops_cross_entropy_finalize
    assert f(None, 2, 4, 64, addr(1), addr(2), addr(3), None) == B.ERR_INVALID_ARG
    assert f(addr(0), 1, 4, 64, addr(1), addr(2), addr(3), None) == B.ERR_INVALID_ARG   # ld < 2T
    assert f(addr(0), 2, 0, 64, addr(1), addr(2), addr(3), None) == B.ERR_INVALID_ARG
    assert f(addr(0), 2, 4, 64, addr(1), addr(2), addr(0), None) == B.ERR_INVALID_ARG   # loss overlaps stats
    assert f(addr(0), 2, 4, 64, addr(1), addr(2), addr(3, 2), None) == B.ERR_MISALIGNED


def test_op_list_rules():
    gelu, tanh, sw = mkop(B.OP_GELU_ERF), mkop(B.OP_GELU_TANH), mkop(B.OP_SWIGLU)
    res = mkop(B.OP_RESIDUAL_ADD, inp=addr(5), ld=64)
    assert lin(ops=[gelu, res]) == B.ERR_INVALID_ARG          # not canonical order
    assert lin(ops=[gelu, gelu]) == B.ERR_INVALID_ARG         # repeated kind
    assert lin(ops=[gelu, tanh]) == B.ERR_INVALID_ARG         # two activations
    assert lin(ops=[gelu, sw]) == B.ERR_INVALID_ARG
    assert lin(ops=[mkop(0)]) == B.ERR_INVALID_ARG            # unknown kind
    assert lin(ops=[mkop(13)]) == B.ERR_INVALID_ARG
    assert lin(ops=[mkop(B.OP_GELU_ERF, reserved=1)]) == B.ERR_INVALID_ARG
    assert lin(ops=[mkop(B.OP_RESIDUAL_ADD, ld=64)]) == B.ERR_INVALID_ARG      # no input
    assert lin(ops=[mkop(B.OP_RESIDUAL_ADD, inp=addr(5), ld=8)]) == B.ERR_INVALID_ARG  # ld < N
    assert lin(ops=[mkop(B.OP_STORE_AUX, dtype=B.F8E4M3, out=addr(5), ld=64)]) == B.ERR_INVALID_ARG
    assert lin(ops=[mkop(B.OP_ROWSUMSQ_PARTIAL, dtype=B.F32, out=addr(5), ld=0)]) == B.ERR_INVALID_ARG
    assert lin(ops=[mkop(B.OP_COL_SCALE)]) == B.ERR_INVALID_ARG
    assert lin(ops=[mkop(B.OP_ROW_SCALE, dtype=B.F32)]) == B.ERR_INVALID_ARG
    arr, n = B.op_array([gelu])
    assert B.lib.fusedops_linear_epilogue(addr(0), 64, addr(1), 64, None, 32, 64, 64, B.BF16, None, 1,
                                          addr(2), 64, B.BF16, None, 0, None) == B.ERR_INVALID_ARG
    assert B.lib.fusedops_linear_epilogue(addr(0), 64, addr(1), 64, None, 32, 64, 64, B.BF16, arr, -1,
                                          addr(2), 64, B.BF16, None, 0, None) == B.ERR_INVALID_ARG


def test_split_rules():
    good = mkop(B.OP_SPLIT_COLS, out_v=[addr(3), addr(4), addr(5)], n_split=3, ld=64)
    assert lin(N=192, ops=[good], Y=addr(2)) == B.ERR_INVALID_ARG   # Y must be NULL
    assert lin(N=192, ops=[mkop(B.OP_SPLIT_COLS, out_v=[addr(3), addr(4), addr(5)], n_split=4, ld=64)],
               Y=None) == B.ERR_INVALID_ARG
    assert lin(N=192, ops=[mkop(B.OP_SPLIT_COLS, out_v=[addr(3), None, addr(5)], n_split=3, ld=64)],
               Y=None) == B.ERR_INVALID_ARG
    assert lin(N=64, ops=[mkop(B.OP_SPLIT_COLS, out_v=[addr(3), addr(4), addr(5)], n_split=3, ld=64)],
               Y=None) == B.ERR_INVALID_ARG   # 64 not divisible by 3
    assert lin(N=96, ops=[mkop(B.OP_SPLIT_COLS, out_v=[addr(3), addr(4), addr(5)], n_split=3, ld=24)],
               Y=None) == B.ERR_INVALID_ARG   # ld < block width 32
    assert lin(N=96, ops=[mkop(B.OP_SPLIT_COLS, out_v=[addr(3), addr(4), addr(5)], n_split=3, ld=36)],
               Y=None) == B.ERR_MISALIGNED    # 72-byte rows
    assert lin(N=96, ops=[mkop(B.OP_SPLIT_COLS, out_v=[addr(3), addr(4, 8), addr(5)], n_split=3, ld=32)],
               Y=None) == B.ERR_MISALIGNED
    assert lin(N=96, ops=[mkop(B.OP_SPLIT_COLS, out_v=[addr(3), addr(3, 64), addr(5)], n_split=3, ld=32)],
               Y=None) == B.ERR_INVALID_ARG   # two blocks overlap


def test_alignment_rules():
    assert lin(K=60, ldx=64, ldw=64) == B.ERR_MISALIGNED            # K % 8 (bf16)
    assert lin(N=61, ldy=61) == B.ERR_MISALIGNED                    # Y rows not 16-byte aligned
    # any N: N = 61 passes the alignment checks and fails only at the later workspace check
    q = mkop(B.OP_QUANT_FP8_ROW, dtype=B.F32, out=addr(6))
    assert lin(N=61, ldy=64, ops=[q], out_dt=B.F8E4M3) == B.ERR_WORKSPACE
    assert lin(X=addr(0, 8)) == B.ERR_MISALIGNED
    assert lin(W=addr(1, 2)) == B.ERR_MISALIGNED
    assert lin(Y=addr(2, 4)) == B.ERR_MISALIGNED
    assert lin(ldx=68) == B.ERR_MISALIGNED                          # row stride not 16 bytes
    assert lin(ldy=68) == B.ERR_MISALIGNED
    assert lin(bias=addr(6, 8)) == B.ERR_MISALIGNED
    assert lin(in_dt=B.F32, K=62, ldx=64, ldw=64, out_dt=B.F32) == B.ERR_MISALIGNED  # K % 4 (fp32)
    res = mkop(B.OP_RESIDUAL_ADD, inp=addr(5, 8), ld=64)
    assert lin(ops=[res]) == B.ERR_MISALIGNED
    par = mkop(B.OP_ROWSUMSQ_PARTIAL, dtype=B.F32, out=addr(5, 2), ld=1)
    assert lin(ops=[par]) == B.ERR_MISALIGNED


def test_quant_rules_and_workspace():
    q = mkop(B.OP_QUANT_FP8_ROW, dtype=B.F32, out=addr(6))
    sw = mkop(B.OP_SWIGLU)
    assert lin(ops=[sw, q], ldy=32, out_dt=B.BF16) == B.ERR_INVALID_ARG      # needs fp8 out
    assert lin(ops=[sw, q], ldy=32, out_dt=B.F8E4M3) == B.ERR_WORKSPACE       # no workspace
    need = B.fusedops_linear_workspace_bytes(32, 64, 64, [sw, q])
    assert need > 0 and need % 256 == 0
    assert need >= 4 * (2 + 2 * 1 + 32)
    assert lin(ops=[sw, q], ldy=32, out_dt=B.F8E4M3, ws=addr(7), ws_bytes=need - 4) == B.ERR_WORKSPACE
    assert lin(ops=[sw, q], ldy=32, out_dt=B.F8E4M3, ws=addr(7, 2), ws_bytes=need) == B.ERR_WORKSPACE
    assert lin(ops=[sw, q], ldy=30, out_dt=B.F8E4M3, ws=addr(7), ws_bytes=need) == B.ERR_INVALID_ARG
    assert lin(ops=[sw, q], ldy=40, out_dt=B.F8E4M3, ws=addr(7), ws_bytes=need) == B.ERR_MISALIGNED
    # workspace overlapping an output
    assert lin(ops=[sw, q], ldy=32, out_dt=B.F8E4M3, ws=addr(2), ws_bytes=need) == B.ERR_INVALID_ARG
    assert B.fusedops_linear_workspace_bytes(32, 64, 64, [sw]) == 0
    assert B.fusedops_linear_workspace_bytes(32, 64, 64, [q, sw]) == 0   # invalid list -> 0
    assert B.fusedops_linear_workspace_bytes(0, 64, 64, [sw, q]) == 0


def test_quant_workspace_limit():
    """The kernels address the FP8 workspace in 32 bits: a call that would need more than
    4 GiB of it is refused as unsupported (here M = 2^20 tokens, N = 2^17 features: about
    4 M N / 64 bytes = 8 GiB), before anything is enqueued."""
    M, N, K = 1 << 20, 1 << 17, 64
    q = mkop(B.OP_QUANT_FP8_ROW, dtype=B.F32, out=addr(6))
    sw = mkop(B.OP_SWIGLU)
    need = B.fusedops_linear_workspace_bytes(M, N, K, [sw, q])
    assert need > (1 << 32)
    assert lin(X=addr(0), W=addr(1), M=M, N=N, K=K, ops=[sw, q], Y=addr(16), ldy=N // 2, out_dt=B.F8E4M3,
               ws=addr(40), ws_bytes=need) == B.ERR_UNSUPPORTED
    # a quarter of the tokens fits
    need_q = B.fusedops_linear_workspace_bytes(M // 4, N, K, [sw, q])
    assert 0 < need_q < (1 << 32)


def test_rendezvous_error_rules():
    err = ctypes.c_int32(7)
    assert B.lib.fusedops_rendezvous_error(addr(7), 0, None, None) == B.ERR_INVALID_ARG
    assert B.lib.fusedops_rendezvous_error(None, 0, None, None) == B.ERR_INVALID_ARG
    assert B.lib.fusedops_rendezvous_error(addr(7, 4), 0, ctypes.byref(err), None) == B.ERR_MISALIGNED
    assert err.value == 7   # untouched on an argument error


def test_noalloc_size_limit_and_plain_rules():
    """The allocation-free entry point refuses a quantised call whose rendezvous state would not
    fit its device array, before any HIP call; its other argument checks are the regular ones."""
    q = mkop(B.OP_QUANT_FP8_ROW, dtype=B.F32, out=addr(6))
    sw = mkop(B.OP_SWIGLU)
    M, N, K = 1 << 15, 1 << 15, 64
    assert B.fusedops_linear_workspace_bytes(M, N, K, [sw, q]) > B.NOALLOC_SCRATCH_BYTES
    arr, n = B.op_array([sw, q])
    st = B.lib.fusedops_linear_epilogue_noalloc(addr(0), K, addr(1), K, None, M, N, K, B.BF16, arr, n, addr(2),
                                                N // 2, B.F8E4M3, None)
    assert st == B.ERR_WORKSPACE
    # no quantisation: the regular checks, nothing looked up (invalid leading dimension, null X)
    arr, n = B.op_array([mkop(B.OP_GELU_ERF)])
    assert B.lib.fusedops_linear_epilogue_noalloc(addr(0), 32, addr(1), 64, None, 32, 64, 64, B.BF16, arr, n,
                                                  addr(2), 64, B.BF16, None) == B.ERR_INVALID_ARG
    assert B.lib.fusedops_linear_epilogue_noalloc(None, 64, addr(1), 64, None, 32, 64, 64, B.BF16, arr, n,
                                                  addr(2), 64, B.BF16, None) == B.ERR_INVALID_ARG


def test_aliasing_rules():
    # Y inside X
    assert lin(Y=addr(0, 64)) == B.ERR_INVALID_ARG
    # Y overlapping W
    assert lin(Y=addr(1)) == B.ERR_INVALID_ARG
    # STORE_AUX overlapping Y
    aux = mkop(B.OP_STORE_AUX, out=addr(2, 128), ld=64)
    assert lin(ops=[aux]) == B.ERR_INVALID_ARG
    # residual that overlaps Y without being exactly Y
    res = mkop(B.OP_RESIDUAL_ADD, inp=addr(2, 16), ld=64)
    assert lin(ops=[res]) == B.ERR_INVALID_ARG
    # exact alias with a different stride is not the allowed in-place form
    res2 = mkop(B.OP_RESIDUAL_ADD, inp=addr(2), ld=128)
    assert lin(ops=[res2], ldy=64) == B.ERR_INVALID_ARG
    # partials overlapping the residual input
    res3 = mkop(B.OP_RESIDUAL_ADD, inp=addr(5), ld=64)
    par = mkop(B.OP_ROWSUMSQ_PARTIAL, dtype=B.F32, out=addr(5, 64), ld=1)
    assert lin(ops=[res3, par]) == B.ERR_INVALID_ARG


def ln(x=addr(0), ldx=4096, y=addr(1), ldy=4096, rows=8, cols=4096, io=B.F16, out=B.F16, g=addr(2),
       b=addr(3), pd=B.F16, eps=1e-5, form=B.GELU_TANH):
    return B.lib.fusedops_layernorm_gelu(x, ldx, y, ldy, rows, cols, io, out, g, b, pd, eps, form, None)


def test_layernorm_rules():
    assert ln(x=None) == B.ERR_INVALID_ARG
    assert ln(y=None) == B.ERR_INVALID_ARG
    assert ln(rows=0) == B.ERR_INVALID_ARG
    assert ln(cols=0) == B.ERR_INVALID_ARG
    assert ln(io=5) == B.ERR_INVALID_ARG
    assert ln(io=B.F8E4M3) == B.ERR_UNSUPPORTED
    assert ln(pd=B.F8E4M3) == B.ERR_UNSUPPORTED
    assert ln(eps=0.0) == B.ERR_INVALID_ARG
    assert ln(eps=float("inf")) == B.ERR_INVALID_ARG
    assert ln(eps=float("nan")) == B.ERR_INVALID_ARG
    assert ln(form=3) == B.ERR_INVALID_ARG
    assert ln(ldx=4000) == B.ERR_INVALID_ARG
    assert ln(cols=16392, ldx=16392, ldy=16392) == B.ERR_UNSUPPORTED
    assert ln(cols=3004, ldx=3008, ldy=3008) == B.ERR_MISALIGNED
    assert ln(ldx=4100) == B.ERR_MISALIGNED
    assert ln(x=addr(0, 8)) == B.ERR_MISALIGNED
    assert ln(g=addr(2, 4)) == B.ERR_MISALIGNED
    assert ln(y=addr(0, 16)) == B.ERR_INVALID_ARG    # overlaps x but is not x
    assert ln(y=addr(2)) == B.ERR_INVALID_ARG        # overlaps gamma
    assert ln(io=B.F32, cols=4094, ldx=4096, ldy=4096) == B.ERR_MISALIGNED


def fin(p=addr(0), ldp=16, M=64, T=16, N=2048, eps=1e-6, r=addr(1), h=None, ldh=2048, g=None, y=None,
        ldy=2048, dt=B.BF16):
    return B.lib.fusedops_rmsnorm_finalize(p, ldp, M, T, N, eps, r, h, ldh, g, y, ldy, dt, None)


def test_finalize_rules():
    assert fin(p=None) == B.ERR_INVALID_ARG
    assert fin(r=None) == B.ERR_INVALID_ARG
    assert fin(M=0) == B.ERR_INVALID_ARG
    assert fin(ldp=8) == B.ERR_INVALID_ARG
    assert fin(eps=-1.0) == B.ERR_INVALID_ARG
    assert fin(h=addr(2)) == B.ERR_INVALID_ARG          # h without y
    assert fin(y=addr(3)) == B.ERR_INVALID_ARG          # y without h
    assert fin(p=addr(0, 2)) == B.ERR_MISALIGNED
    assert fin(r=addr(0, 64)) == B.ERR_INVALID_ARG      # r inside the partials
    assert fin(h=addr(2), y=addr(3), dt=9) == B.ERR_INVALID_ARG
    assert fin(h=addr(2), y=addr(3), dt=B.F8E4M3) == B.ERR_UNSUPPORTED
    assert fin(h=addr(2), y=addr(3), ldh=1024) == B.ERR_INVALID_ARG
    assert fin(h=addr(2), y=addr(3), N=2044, ldh=2048) == B.ERR_MISALIGNED
    assert fin(h=addr(2), y=addr(2, 16)) == B.ERR_INVALID_ARG   # y overlaps h, not in place
    assert fin(h=addr(2), y=addr(3), g=addr(3, 32)) == B.ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib.util
    spec = importlib.util.spec_from_file_location("fo_binding_copy",
                                                  os.path.join(ROOT, "gelu_bf16_gemm_amd", "binding.py"))
    mod = importlib.util.module_from_spec(spec)
    src = open(os.path.join(ROOT, "gelu_bf16_gemm_amd", "binding.py")).read()
    src = src.replace('PKG = os.path.dirname(os.path.abspath(__file__))', f'PKG = {str(tmp_path)!r}')
    with pytest.raises(ImportError, match="no CPU fallback"):
        exec(compile(src, "binding_copy", "exec"), mod.__dict__)


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "gelu_bf16_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_single_hip_runtime_in_process():
    """The library must share torch's HIP runtime: exactly one libamdhip64 is mapped."""
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs
