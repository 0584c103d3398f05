"""Thin ctypes binding of libfusedops.so (argument marshalling only).

The functions carry the C names (``fusedops_linear_epilogue`` and friends) and
take torch tensors already on the GPU: they read pointers, leading dimensions
and dtypes, pass the current HIP stream, and return the C status code. They
allocate nothing and compute nothing; every step runs in the HIP kernels.

Loading fails loudly (ImportError) when the library has not been built: there
is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
import struct

# torch brings its own HIP runtime (libamdhip64.so.7). Import it before loading the library so
# that the library's libamdhip64.so.7 dependency resolves to that already-loaded runtime: one
# process must not hold two HIP runtimes (device memory from one is unknown to the other).
import torch  # noqa: F401

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfusedops.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first with `python -m gelu_bf16_gemm_amd.build` "
        "(the fused-linear path has no CPU fallback)")

lib = ctypes.CDLL(LIB_PATH)

# status codes / enums (mirror include/fusedops.h)
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_WORKSPACE, ERR_LAUNCH = 0, -1, -2, -3, -4, -5
F32, BF16, F16, F8E4M3 = 0, 1, 2, 3
(OP_RESIDUAL_ADD, OP_STORE_AUX, OP_ROWSUMSQ_PARTIAL, OP_COL_SCALE, OP_ROW_SCALE, OP_GELU_ERF,
 OP_GELU_TANH, OP_SWIGLU, OP_QUANT_FP8_ROW, OP_SPLIT_COLS, OP_DEQUANT_ROW, OP_DEQUANT_COL, OP_ROPE,
 OP_ROW_RMS, OP_XENT) = range(1, 16)
GELU_NONE, GELU_TANH, GELU_ERF = 0, 1, 2
PARTIAL_COLS = 128
XENT_COLS = 64
LN_MAX_COLS = 16384

# every symbol the public header declares
EXPORTS = ("fusedops_linear_epilogue", "fusedops_linear_workspace_bytes", "fusedops_layernorm_gelu",
           "fusedops_rmsnorm_finalize", "fusedops_cross_entropy_finalize", "fusedops_partial_cols",
           "fusedops_abi_version", "fusedops_status_string", "fusedops_rendezvous_error",
           "fusedops_linear_epilogue_noalloc")
NOALLOC_SCRATCH_BYTES = 32 << 20


class Op(ctypes.Structure):
    """struct fusedops_op (64 bytes)."""
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("in_", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("ld", ctypes.c_int64), ("out_v", ctypes.c_void_p * 3),
                ("n_split", ctypes.c_int32), ("reserved", ctypes.c_int32)]


assert ctypes.sizeof(Op) == 64

_i64, _i32, _vp, _f32, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t

lib.fusedops_linear_epilogue.restype = _i32
lib.fusedops_linear_epilogue.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32,
                                         ctypes.POINTER(Op), _i32, _vp, _i64, _i32, _vp, _sz, _vp]
lib.fusedops_linear_epilogue_noalloc.restype = _i32
lib.fusedops_linear_epilogue_noalloc.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32,
                                                 ctypes.POINTER(Op), _i32, _vp, _i64, _i32, _vp]
lib.fusedops_linear_workspace_bytes.restype = _sz
lib.fusedops_linear_workspace_bytes.argtypes = [_i64, _i64, _i64, ctypes.POINTER(Op), _i32]
lib.fusedops_layernorm_gelu.restype = _i32
lib.fusedops_layernorm_gelu.argtypes = [_vp, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _i32,
                                        _f32, _i32, _vp]
lib.fusedops_rmsnorm_finalize.restype = _i32
lib.fusedops_rmsnorm_finalize.argtypes = [_vp, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _i64, _vp,
                                          _vp, _i64, _i32, _vp]
lib.fusedops_cross_entropy_finalize.restype = _i32
lib.fusedops_cross_entropy_finalize.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
lib.fusedops_rendezvous_error.restype = _i32
lib.fusedops_rendezvous_error.argtypes = [_vp, _i32, ctypes.POINTER(_i32), _vp]
lib.fusedops_partial_cols.restype = _i32
lib.fusedops_partial_cols.argtypes = []
lib.fusedops_abi_version.restype = _i32
lib.fusedops_abi_version.argtypes = []
lib.fusedops_status_string.restype = ctypes.c_char_p
lib.fusedops_status_string.argtypes = [_i32]


class FusedOpsError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"fusedops status {status}: {lib.fusedops_status_string(status).decode()}")


def check(status: int) -> None:
    if status != OK:
        raise FusedOpsError(status)


# ---------------------------------------------------------------------------
# torch marshalling helpers
# ---------------------------------------------------------------------------

def dtype_code(t) -> int:
    m = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16, torch.uint8: F8E4M3}
    if hasattr(torch, "float8_e4m3fn"):
        m[torch.float8_e4m3fn] = F8E4M3
    return m[t.dtype]


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _ld(t) -> int:
    if t.dim() == 1:
        return t.shape[0]
    if t.stride(-1) != 1:
        raise ValueError("columns must be contiguous")
    return t.stride(0)


def _stream(stream) -> int | None:
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream


def op(kind: int, tensor=None, *, out=None, split=None, head_dim=None) -> Op:
    """Build one epilogue op. `tensor` is the op's input (z, gamma, r, scales, RoPE table) and
    `out` its output (h1, partials, scales); `split` is the list of SPLIT_COLS destination
    tensors; `head_dim` is ROPE's head width d."""
    o = Op()
    o.kind = kind
    t = tensor if tensor is not None else out
    if t is not None:
        o.dtype = dtype_code(t)
        o.ld = _ld(t)
    if tensor is not None:
        o.in_ = tensor.data_ptr()
    if out is not None:
        o.out = out.data_ptr()
    if split is not None:
        o.n_split = len(split)
        o.ld = _ld(split[0])
        o.dtype = dtype_code(split[0])
        for i, s in enumerate(split):
            o.out_v[i] = s.data_ptr()
    if head_dim is not None:
        o.n_split = head_dim
    # the op holds raw device pointers: keep their tensors alive as long as the op
    o.tensors = tuple(t for t in (tensor, out, *(split or ())) if t is not None)
    return o


def row_rms_op(partials, width: int, eps: float) -> Op:
    """ROW_RMS: the deferred RMSNorm row scale from a previous call's row partials."""
    o = op(OP_ROW_RMS, partials)
    o.n_split = width
    o.reserved = int.from_bytes(struct.pack("<f", eps), "little", signed=True)
    return o


def op_array(ops) -> tuple:
    arr = (Op * max(1, len(ops)))(*ops) if ops else (Op * 1)()
    return arr, len(ops)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def fusedops_linear_workspace_bytes(M: int, N: int, K: int, ops=()) -> int:
    arr, n = op_array(list(ops))
    return lib.fusedops_linear_workspace_bytes(M, N, K, arr, n)


def fusedops_linear_epilogue(x, w, y, *, bias=None, ops=(), workspace=None, out_dtype=None,
                             stream=None) -> int:
    """Y = epilogue(X W^T + b); x (M,K), w (N,K), y (M, N_out) or None with SPLIT_COLS."""
    M, K = x.shape
    N = w.shape[0]
    arr, n = op_array(list(ops))
    od = out_dtype if out_dtype is not None else (dtype_code(y) if y is not None else None)
    if od is None:
        split = [o for o in ops if o.kind == OP_SPLIT_COLS]
        od = split[0].dtype if split else F32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return lib.fusedops_linear_epilogue(
        x.data_ptr(), _ld(x), w.data_ptr(), _ld(w), _ptr(bias), M, N, K, dtype_code(x), arr, n,
        _ptr(y), _ld(y) if y is not None else 0, od, _ptr(workspace), ws_bytes, _stream(stream))


def fusedops_linear_epilogue_noalloc(x, w, y, *, bias=None, ops=(), out_dtype=None, stream=None) -> int:
    """fusedops_linear_epilogue without a workspace: FP8 rendezvous state in the library's
    per-GPU device array (for callers that cannot allocate)."""
    M, K = x.shape
    N = w.shape[0]
    arr, n = op_array(list(ops))
    od = out_dtype if out_dtype is not None else (dtype_code(y) if y is not None else None)
    if od is None:
        split = [o for o in ops if o.kind == OP_SPLIT_COLS]
        od = split[0].dtype if split else F32
    return lib.fusedops_linear_epilogue_noalloc(
        x.data_ptr(), _ld(x), w.data_ptr(), _ld(w), _ptr(bias), M, N, K, dtype_code(x), arr, n,
        _ptr(y), _ld(y) if y is not None else 0, od, _stream(stream))


def prepare_linear_epilogue(x, w, y, *, bias=None, ops=(), workspace=None, out_dtype=None, stream=None):
    """The arguments of one fusedops_linear_epilogue call, marshalled once; the returned function
    makes exactly that call and returns its status. For launch loops, where marshalling every
    call would take longer than a small kernel runs. The stream is the one current now unless
    given; the tensors must stay alive and unchanged in shape while the function is used."""
    M, K = x.shape
    N = w.shape[0]
    arr, n = op_array(list(ops))
    od = out_dtype if out_dtype is not None else (dtype_code(y) if y is not None else None)
    if od is None:
        split = [o for o in ops if o.kind == OP_SPLIT_COLS]
        od = split[0].dtype if split else F32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (x.data_ptr(), _ld(x), w.data_ptr(), _ld(w), _ptr(bias), M, N, K, dtype_code(x), arr, n,
            _ptr(y), _ld(y) if y is not None else 0, od, _ptr(workspace), ws_bytes, _stream(stream))
    fn = lib.fusedops_linear_epilogue

    def call() -> int:
        return fn(*args)

    # the buffers, the ops (which hold their own tensors) and the op array live as long as call
    call.keep = (x, w, y, bias, workspace, tuple(ops), arr)
    return call


def fusedops_layernorm_gelu(x, y, gamma=None, beta=None, *, eps: float = 1e-5, gelu_form: int = GELU_TANH,
                            stream=None) -> int:
    rows, cols = x.shape
    pd = dtype_code(gamma) if gamma is not None else (dtype_code(beta) if beta is not None else F32)
    return lib.fusedops_layernorm_gelu(x.data_ptr(), _ld(x), y.data_ptr(), _ld(y), rows, cols,
                                       dtype_code(x), dtype_code(y), _ptr(gamma), _ptr(beta), pd,
                                       eps, gelu_form, _stream(stream))


def fusedops_rmsnorm_finalize(partials, n_cols: int, eps: float, r, *, h=None, gamma=None, y=None,
                              stream=None) -> int:
    M, T = partials.shape
    dt = dtype_code(h) if h is not None else F32
    return lib.fusedops_rmsnorm_finalize(
        partials.data_ptr(), _ld(partials), M, T, n_cols, eps, r.data_ptr(), _ptr(h),
        _ld(h) if h is not None else 0, _ptr(gamma), _ptr(y), _ld(y) if y is not None else 0, dt,
        _stream(stream))


def xent_op(labels, stats, target) -> Op:
    """XENT: labels (int32, M), stats (fp32, M x 2T), target (fp32, M)."""
    o = Op()
    o.kind = OP_XENT
    o.dtype = F32
    o.in_ = labels.data_ptr()
    o.out = stats.data_ptr()
    o.ld = _ld(stats)
    o.out_v[0] = target.data_ptr()
    o.tensors = (labels, stats, target)
    return o


def fusedops_cross_entropy_finalize(stats, n_cols: int, target, labels, loss, *, stream=None) -> int:
    M = stats.shape[0]
    return lib.fusedops_cross_entropy_finalize(stats.data_ptr(), _ld(stats), M, n_cols, target.data_ptr(),
                                               labels.data_ptr(), loss.data_ptr(), _stream(stream))


def fusedops_rendezvous_error(workspace, *, clear: bool = False, stream=None) -> tuple:
    """(status, error word 0 / 1) of an FP8 workspace; synchronises the stream."""
    err = _i32(-1)
    st = lib.fusedops_rendezvous_error(_ptr(workspace), 1 if clear else 0, ctypes.byref(err), _stream(stream))
    return st, err.value


def abi_version() -> int:
    return lib.fusedops_abi_version()


def partial_cols() -> int:
    return lib.fusedops_partial_cols()


def status_string(s: int) -> str:
    return lib.fusedops_status_string(s).decode()
