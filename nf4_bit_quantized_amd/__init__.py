"""Python binding of the MI355X QLoRA NF4 linear-layer library.

Argument marshalling only: each function here has the name of a C entry point
declared in ``include/qlora.h``, checks and converts its arguments (torch
tensors on the GPU, the current stream), allocates missing outputs and
workspace with torch, and calls the entry point through ctypes.  Every step of
the layer runs in the library's HIP kernels.  If the library is not built, or
no GPU is present when a compute call is made, an error is raised: there is no
fallback implementation.

The library loaded is ``libqlora_nf4.so`` next to this file, or the file that
the environment variable ``QLORA_NF4_LIBRARY`` names (for example a build of
the same sources with host-side sanitizers).
"""

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("QLORA_NF4_LIBRARY") or os.path.join(HERE, "libqlora_nf4.so")

QLORA_OK = 0
QLORA_ERR_NULL = -1
QLORA_ERR_SHAPE = -2
QLORA_ERR_UNSUPPORTED = -3
QLORA_ERR_WORKSPACE = -4
QLORA_ERR_HIP = -5
QLORA_ERR_SCRATCH_LIMIT = -6

# device bytes of the library's static scratch array (qlora_linear_fwd_noalloc)
QLORA_STATIC_SCRATCH_BYTES = 16 << 20

# element formats of the weight handed to quantization
QLORA_W_F32 = 0
QLORA_W_BF16 = 1
QLORA_W_F16 = 2

# Every exported symbol of include/qlora.h
EXPORTED = (
    "qlora_status_string",
    "qlora_nf4_levels",
    "qlora_table_levels",
    "qlora_nf4_sizes",
    "qlora_quantize_nf4",
    "qlora_quantize_nf4_typed",
    "qlora_fwd_workspace_bytes",
    "qlora_linear_fwd",
    "qlora_linear_fwd_noalloc",
    "qlora_bwd_workspace_bytes",
    "qlora_linear_bwd",
    "qlora_linear_bwd_accumulate",
    "qlora_dropout_workspace_bytes",
    "qlora_linear_fwd_dropout",
    "qlora_linear_bwd_dropout",
    "qlora_multi_fwd_workspace_bytes",
    "qlora_linear_fwd_multi",
    "qlora_multi_bwd_workspace_bytes",
    "qlora_linear_bwd_multi",
    "qlora_dequantize_nf4",
    "qlora_merge_lora",
    "qlora_adamw_step",
    "qlora_trace_enable",
    "qlora_trace_select",
    "qlora_trace_kernel_name",
    "qlora_trace_read",
)


class QloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({qlora_status_string(status)})")


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class Nf4Desc(ctypes.Structure):
    _fields_ = [("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64),
                ("blocksize", ctypes.c_int32), ("dq_blocksize", ctypes.c_int32), ("table", ctypes.c_int32)]


class AdamwHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("grad_scale", ctypes.c_float),
                ("step", ctypes.c_int64)]


# level tables (qlora_nf4_desc.table)
TABLE_NF4 = 0
TABLE_UNIFORM = 1


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} missing "
                           "(run python -m nf4_bit_quantized_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i64, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    dp = ctypes.POINTER(Nf4Desc)
    L.qlora_status_string.argtypes = [ctypes.c_int]
    L.qlora_status_string.restype = ctypes.c_char_p
    L.qlora_nf4_levels.argtypes = [vp, vp]
    L.qlora_table_levels.argtypes = [i32, vp, vp]
    L.qlora_nf4_sizes.argtypes = [dp, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.qlora_quantize_nf4.argtypes = [dp, vp, vp, vp, vp, vp]
    L.qlora_quantize_nf4_typed.argtypes = [dp, vp, i32, vp, vp, vp, vp]
    L.qlora_fwd_workspace_bytes.argtypes = [dp, i64, i32, ctypes.POINTER(sz)]
    L.qlora_bwd_workspace_bytes.argtypes = [dp, i64, i32, ctypes.POINTER(sz)]
    L.qlora_linear_fwd.argtypes = [dp, vp, vp, vp, i64, vp, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    L.qlora_linear_fwd_noalloc.argtypes = [dp, vp, vp, vp, i64, vp, i32, f32, vp, vp, vp, vp, vp]
    L.qlora_linear_bwd.argtypes = [dp, vp, vp, vp, i64, vp, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.qlora_linear_bwd_accumulate.argtypes = L.qlora_linear_bwd.argtypes
    L.qlora_dropout_workspace_bytes.argtypes = [dp, i64, i32, i32, ctypes.POINTER(sz)]
    L.qlora_multi_fwd_workspace_bytes.argtypes = [i32, dp, i64, i32, ctypes.POINTER(sz)]
    L.qlora_linear_fwd_multi.argtypes = [i32, dp, vp, vp, vp, i64, vp, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    L.qlora_multi_bwd_workspace_bytes.argtypes = [i32, dp, i64, i32, ctypes.POINTER(sz)]
    L.qlora_linear_bwd_multi.argtypes = [i32, dp, vp, vp, vp, i64, vp, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.qlora_linear_fwd_dropout.argtypes = [dp, vp, vp, vp, i64, vp, i32, f32, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    L.qlora_linear_bwd_dropout.argtypes = [dp, vp, vp, vp, i64, vp, i32, f32, vp, vp, vp, vp, vp, f32, vp, vp, vp,
                                           i32, vp, sz, vp]
    L.qlora_dequantize_nf4.argtypes = [dp, vp, vp, vp, vp, vp]
    L.qlora_merge_lora.argtypes = [dp, vp, vp, vp, i32, f32, vp, vp, vp, vp]
    L.qlora_adamw_step.argtypes = [ctypes.POINTER(AdamwHparams), i64, vp, vp, vp, vp, vp, vp]
    L.qlora_trace_enable.argtypes = [ctypes.c_int]
    L.qlora_trace_select.argtypes = [ctypes.c_uint32]
    L.qlora_trace_kernel_name.argtypes = [ctypes.c_int]
    L.qlora_trace_read.argtypes = [ctypes.POINTER(KernelStat), ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                   ctypes.c_int]
    for name in EXPORTED[1:]:
        getattr(L, name).restype = ctypes.c_int
    L.qlora_trace_kernel_name.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int, where: str):
    if status != QLORA_OK:
        raise QloraError(status, where)


def _desc(d_out: int, d_in: int, blocksize: int = 64, dq_blocksize: int = 256, table: int = TABLE_NF4) -> Nf4Desc:
    return Nf4Desc(int(d_out), int(d_in), int(blocksize), int(dq_blocksize), int(table))


def _stored_desc(packed, codes, consts, table: int) -> Nf4Desc:
    """Descriptor of a stored weight.  Its block size follows from the length
    of its codes array (one code per block); an empty codes array means no
    second level, and consts then holds one fp32 scale per block."""
    d_out, d_in = packed.shape[0], packed.shape[1] * 2
    dq = codes is not None and codes.numel() > 0
    nb = codes.numel() if dq else consts.numel()
    if nb <= 0 or (d_out * d_in) % nb != 0 or (d_out * d_in) // nb not in (64, 128, 256):
        raise ValueError(f"{'codes' if dq else 'consts'} holds {nb} entries: not one per block of 64, 128 or "
                         f"256 weights of a {d_out}x{d_in} weight")
    bs = (d_out * d_in) // nb
    want_k = -(-nb // 256) if dq else nb
    if consts.numel() != want_k:
        raise ValueError(f"consts holds {consts.numel()} entries, expected {want_k}")
    return _desc(d_out, d_in, bs, 256 if dq else 0, table=table)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need_cuda(*tensors, dtype=None, name=""):
    import torch
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name}: tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensors must be contiguous")


def _check_out(t, shape, dtype, name: str):
    """A caller-given output: contiguous, of the shape and dtype the call writes."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def _check_in(t, shape, dtype, name: str):
    """A required input: of the shape and dtype the weight's descriptor and the
    call imply, contiguous.  The kernels size their reads from the stored
    weight's shape, so a smaller tensor would be read past its end."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def _matrix(X, name: str = "X"):
    """X must be a 2-D tensor (its rows are the tokens)."""
    if X is None or X.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    return X


def _check_weight(packed, codes, consts, name: str = "weight"):
    """The stored weight: packed uint8 [d_out][d_in/2], codes uint8 and
    consts float32 (one-dimensional, contiguous)."""
    import torch
    if packed is None or consts is None:
        raise ValueError(f"{name}: packed and consts are required")
    if packed.dtype != torch.uint8 or packed.dim() != 2 or not packed.is_contiguous():
        raise ValueError(f"{name}: packed must be a contiguous 2-D uint8 tensor")
    if codes is not None and (codes.dtype != torch.uint8 or codes.dim() != 1 or not codes.is_contiguous()):
        raise ValueError(f"{name}: codes must be a contiguous 1-D uint8 tensor")
    if consts.dtype != torch.float32 or consts.dim() != 1 or not consts.is_contiguous():
        raise ValueError(f"{name}: consts must be a contiguous 1-D float32 tensor")


def _check_adapter(A, B, d_out: int, d_in: int, r: int, name: str = ""):
    """A bf16 [r][d_in] and B bf16 [d_out][r], both given or both None (r = 0)."""
    import torch
    if (A is None) != (B is None):
        raise ValueError(f"{name}A and B must be given together")
    if A is None:
        return
    _check_in(A, (r, d_in), torch.bfloat16, f"{name}A")
    _check_in(B, (d_out, r), torch.bfloat16, f"{name}B")


# ---------------------------------------------------------------------------
# Host-only queries
# ---------------------------------------------------------------------------

def qlora_status_string(status: int) -> str:
    return lib().qlora_status_string(int(status)).decode()


def qlora_nf4_levels():
    """(levels float32[16], thresholds float32[15]) as numpy arrays."""
    import numpy as np
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    _check(lib().qlora_nf4_levels(ctypes.cast(lv, ctypes.c_void_p), ctypes.cast(th, ctypes.c_void_p)),
           "qlora_nf4_levels")
    return np.frombuffer(lv, dtype=np.float32).copy(), np.frombuffer(th, dtype=np.float32).copy()


def qlora_table_levels(table: int = TABLE_NF4):
    """(levels float32[16], thresholds float32[15]) of level table `table`."""
    import numpy as np
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    _check(lib().qlora_table_levels(int(table), ctypes.cast(lv, ctypes.c_void_p), ctypes.cast(th, ctypes.c_void_p)),
           "qlora_table_levels")
    return np.frombuffer(lv, dtype=np.float32).copy(), np.frombuffer(th, dtype=np.float32).copy()


def qlora_nf4_sizes(d_out: int, d_in: int, blocksize: int = 64, dq_blocksize: int = 256) -> Tuple[int, int, int]:
    d = _desc(d_out, d_in, blocksize, dq_blocksize)
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().qlora_nf4_sizes(ctypes.byref(d), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "qlora_nf4_sizes")
    return a.value, b.value, c.value


def qlora_fwd_workspace_bytes(d_out: int, d_in: int, T: int, r: int) -> int:
    d = _desc(d_out, d_in)
    n = ctypes.c_size_t()
    _check(lib().qlora_fwd_workspace_bytes(ctypes.byref(d), int(T), int(r), ctypes.byref(n)),
           "qlora_fwd_workspace_bytes")
    return n.value


def qlora_bwd_workspace_bytes(d_out: int, d_in: int, T: int, r: int) -> int:
    d = _desc(d_out, d_in)
    n = ctypes.c_size_t()
    _check(lib().qlora_bwd_workspace_bytes(ctypes.byref(d), int(T), int(r), ctypes.byref(n)),
           "qlora_bwd_workspace_bytes")
    return n.value


def qlora_multi_fwd_workspace_bytes(shapes, T: int, r: int) -> int:
    """Workspace of qlora_linear_fwd_multi for weights of the given
    (d_out, d_in) shapes (blocks of 64, double quantization)."""
    n = len(shapes)
    descs = (Nf4Desc * n)(*[_desc(o, i) for o, i in shapes])
    b = ctypes.c_size_t()
    _check(lib().qlora_multi_fwd_workspace_bytes(n, descs, int(T), int(r), ctypes.byref(b)),
           "qlora_multi_fwd_workspace_bytes")
    return b.value


def qlora_multi_bwd_workspace_bytes(shapes, T: int, r: int) -> int:
    """Workspace of qlora_linear_bwd_multi for weights of the given shapes."""
    n = len(shapes)
    descs = (Nf4Desc * n)(*[_desc(o, i) for o, i in shapes])
    b = ctypes.c_size_t()
    _check(lib().qlora_multi_bwd_workspace_bytes(n, descs, int(T), int(r), ctypes.byref(b)),
           "qlora_multi_bwd_workspace_bytes")
    return b.value


# ---------------------------------------------------------------------------
# Compute calls (enqueue on the current torch stream; no synchronization)
# ---------------------------------------------------------------------------

def _workspace(nbytes: int, device, workspace=None):
    import torch
    if nbytes == 0:
        return workspace
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def qlora_quantize_nf4(W, packed=None, codes=None, consts=None, stream=None, table: int = TABLE_NF4,
                       blocksize: int = 64, double_quant: bool = True):
    """Quantize W [d_out][d_in] (GPU; float32, bfloat16 or float16) ->
    (packed uint8 [d_out][d_in/2], codes uint8 [nb], consts float32 [ng]),
    nb = d_out * d_in / blocksize (64, 128 or 256 weights per absmax block).
    double_quant=False keeps the fp32 block scales: codes is empty and consts
    holds the nb scales.  A 16-bit W is widened exactly to fp32 in the kernel."""
    import torch
    _need_cuda(W, name="qlora_quantize_nf4")
    fmts = {torch.float32: QLORA_W_F32, torch.bfloat16: QLORA_W_BF16, torch.float16: QLORA_W_F16}
    if W.dtype not in fmts or W.dim() != 2:
        raise ValueError("W must be a 2-D float32, bfloat16 or float16 tensor")
    d_out, d_in = W.shape
    dqb = 256 if double_quant else 0
    n_p, n_c, n_k = qlora_nf4_sizes(d_out, d_in, blocksize, dqb)
    if packed is None:
        packed = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=W.device)
    if codes is None:
        codes = torch.empty(n_c, dtype=torch.uint8, device=W.device)
    if consts is None:
        consts = torch.empty(n_k // 4, dtype=torch.float32, device=W.device)
    _need_cuda(packed, codes, consts, name="qlora_quantize_nf4")
    for t, nm, n, dt in ((packed, "packed", n_p, torch.uint8), (codes, "codes", n_c, torch.uint8),
                         (consts, "consts", n_k // 4, torch.float32)):
        if t.dtype != dt or t.numel() != n or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous {dt} tensor of {n} elements")
    d = _desc(d_out, d_in, blocksize, dqb, table=table)
    if W.dtype == torch.float32:
        _check(lib().qlora_quantize_nf4(ctypes.byref(d), _ptr(W), _ptr(packed), _ptr(codes), _ptr(consts),
                                        _stream(stream)), "qlora_quantize_nf4")
    else:
        _check(lib().qlora_quantize_nf4_typed(ctypes.byref(d), _ptr(W), fmts[W.dtype], _ptr(packed), _ptr(codes),
                                              _ptr(consts), _stream(stream)), "qlora_quantize_nf4_typed")
    return packed, codes, consts


def qlora_linear_fwd(packed, codes, consts, X, A, B, alpha: float, Y=None, U_out=None,
                     want_u: bool = True, workspace=None, stream=None, table: int = TABLE_NF4,
                     keep=None, p: float = 0.0):
    """Forward: returns (Y bf16 [T][d_out], U fp32 [T][r] or None).

    ``packed`` [d_out][d_in/2] fixes the layer shape; X bf16 [T][d_in],
    A bf16 [r][d_in], B bf16 [d_out][r] (A, B may be None for r = 0).
    keep (uint8 [T][d_in/8] keep bits) applies LoRA dropout with rate p to
    the adapter's input (qlora_linear_fwd_dropout).
    """
    import torch
    d_out, d_in = packed.shape[0], packed.shape[1] * 2
    _matrix(X)
    T = X.shape[0]
    r = 0 if A is None else A.shape[0]
    _check_weight(packed, codes, consts)
    _check_in(X, (T, d_in), torch.bfloat16, "X")
    _check_adapter(A, B, d_out, d_in, r)
    _need_cuda(packed, codes, consts, X, A, B, Y, U_out, name="qlora_linear_fwd")
    _check_out(Y, (T, d_out), torch.bfloat16, "Y")
    _check_out(U_out, (T, r), torch.float32, "U_out")
    if Y is None:
        Y = torch.empty((T, d_out), dtype=torch.bfloat16, device=X.device)
    if U_out is None and want_u and r > 0:
        U_out = torch.empty((T, r), dtype=torch.float32, device=X.device)
    d = _stored_desc(packed, codes, consts, table)
    if keep is not None:
        _check_keep(keep, T, d_in)
        nbytes = _dropout_ws(d, T, r, 0)
        ws = _workspace(nbytes, X.device, workspace)
        _check(lib().qlora_linear_fwd_dropout(ctypes.byref(d), _ptr(packed), _ptr(codes), _ptr(consts), T, _ptr(X),
                                              r, float(alpha), _ptr(A), _ptr(B), _ptr(keep), float(p), _ptr(Y),
                                              _ptr(U_out), _ptr(ws), nbytes, _stream(stream)),
               "qlora_linear_fwd_dropout")
        return Y, U_out
    nbytes = qlora_fwd_workspace_bytes(d_out, d_in, T, r)
    ws = _workspace(nbytes, X.device, workspace)
    _check(lib().qlora_linear_fwd(ctypes.byref(d), _ptr(packed), _ptr(codes), _ptr(consts), T, _ptr(X), r,
                                  float(alpha), _ptr(A), _ptr(B), _ptr(Y), _ptr(U_out), _ptr(ws), nbytes,
                                  _stream(stream)), "qlora_linear_fwd")
    return Y, U_out


def qlora_linear_fwd_noalloc(packed, codes, consts, X, A, B, alpha: float, Y, U_out=None, stream=None,
                             table: int = TABLE_NF4):
    """The forward through qlora_linear_fwd_noalloc: no workspace and no
    allocation anywhere (the caller gives Y, and U_out if it wants U); the
    library's static per-GPU scratch serves the call.  Calls that may overlap
    on one GPU race on that scratch.  Returns (Y, U_out)."""
    import torch
    _matrix(X)
    d_out, d_in = packed.shape[0], packed.shape[1] * 2
    T = X.shape[0]
    r = 0 if A is None else A.shape[0]
    _check_weight(packed, codes, consts)
    _check_in(X, (T, d_in), torch.bfloat16, "X")
    _check_adapter(A, B, d_out, d_in, r)
    if Y is None:
        raise ValueError("Y is required (this call allocates nothing)")
    _check_out(Y, (T, d_out), torch.bfloat16, "Y")
    _check_out(U_out, (T, r), torch.float32, "U_out")
    _need_cuda(packed, codes, consts, X, A, B, Y, U_out, name="qlora_linear_fwd_noalloc")
    d = _stored_desc(packed, codes, consts, table)
    _check(lib().qlora_linear_fwd_noalloc(ctypes.byref(d), _ptr(packed), _ptr(codes), _ptr(consts), T, _ptr(X), r,
                                          float(alpha), _ptr(A), _ptr(B), _ptr(Y), _ptr(U_out), _stream(stream)),
           "qlora_linear_fwd_noalloc")
    return Y, U_out


def _check_keep(keep, T: int, d_in: int):
    import torch
    if keep.dtype != torch.uint8 or tuple(keep.shape) != (T, d_in // 8) or not keep.is_contiguous():
        raise ValueError(f"keep must be a contiguous uint8 tensor of shape {(T, d_in // 8)}")
    _need_cuda(keep, name="keep")


def _dropout_ws(d, T: int, r: int, backward: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().qlora_dropout_workspace_bytes(ctypes.byref(d), int(T), int(r), int(backward), ctypes.byref(n)),
           "qlora_dropout_workspace_bytes")
    return n.value


def qlora_linear_fwd_multi(layers, X, alpha: float, want_u: bool = True, workspace=None, stream=None,
                           tables=None, outs=None):
    """Forward of up to four layers sharing X: ``layers`` is a list of
    (packed, codes, consts, A, B) (A, B None for r = 0, the same r for all).
    ``outs`` optionally gives each layer's (Y, U) buffers (U may be None);
    with them and ``workspace`` the call allocates nothing.
    Returns a list of (Y, U) as qlora_linear_fwd does for each layer."""
    import torch
    n = len(layers)
    if not 1 <= n <= 4:
        raise ValueError("one to four layers")
    _matrix(X)
    T = X.shape[0]
    r = 0 if layers[0][3] is None else layers[0][3].shape[0]
    tables = tables or [TABLE_NF4] * n
    if outs is not None and len(outs) != n:
        raise ValueError("one (Y, U) pair per layer")
    given, outs = outs, []
    descs = (Nf4Desc * n)()
    _check_in(X, (T, X.shape[1]), torch.bfloat16, "X")
    for i, (packed, codes, consts, A, B) in enumerate(layers):      # every layer's shapes first
        _check_weight(packed, codes, consts, f"layers[{i}]")
        if packed.shape[1] * 2 != X.shape[1]:
            raise ValueError(f"layers[{i}]: d_in {packed.shape[1] * 2} differs from X's {X.shape[1]}")
        _check_adapter(A, B, packed.shape[0], X.shape[1], r, f"layers[{i}] ")
    for i, (packed, codes, consts, A, B) in enumerate(layers):
        _need_cuda(packed, codes, consts, A, B, name="qlora_linear_fwd_multi")
        descs[i] = _stored_desc(packed, codes, consts, tables[i])
        if given is not None:
            Y, U = given[i]
            _check_out(Y, (T, packed.shape[0]), torch.bfloat16, f"outs[{i}] Y")
            _check_out(U, (T, r), torch.float32, f"outs[{i}] U")
            _need_cuda(Y, U, name="qlora_linear_fwd_multi")
            if Y is None:
                raise ValueError(f"outs[{i}]: Y is required")
        else:
            Y = torch.empty((T, packed.shape[0]), dtype=torch.bfloat16, device=X.device)
            U = torch.empty((T, r), dtype=torch.float32, device=X.device) if want_u and r > 0 else None
        outs.append((Y, U))
    _need_cuda(X, name="qlora_linear_fwd_multi")
    n_b = ctypes.c_size_t()
    _check(lib().qlora_multi_fwd_workspace_bytes(n, descs, int(T), int(r), ctypes.byref(n_b)),
           "qlora_multi_fwd_workspace_bytes")
    ws = _workspace(n_b.value, X.device, workspace)
    arr = lambda vals: (ctypes.c_void_p * n)(*vals)
    _check(lib().qlora_linear_fwd_multi(
        n, descs, arr([_ptr(l[0]) for l in layers]), arr([_ptr(l[1]) for l in layers]),
        arr([_ptr(l[2]) for l in layers]), int(T), _ptr(X), int(r), float(alpha),
        arr([_ptr(l[3]) for l in layers]), arr([_ptr(l[4]) for l in layers]), arr([_ptr(o[0]) for o in outs]),
        arr([_ptr(o[1]) for o in outs]), _ptr(ws), n_b.value, _stream(stream)), "qlora_linear_fwd_multi")
    return outs


def qlora_linear_bwd_multi(layers, X, alpha: float, dYs, U_ins=None, want_dx: bool = True, workspace=None,
                           stream=None, tables=None, dX=None, grads=None):
    """Backward of up to four layers sharing X: ``layers`` as for
    qlora_linear_fwd_multi, ``dYs`` each layer's upstream gradient, ``U_ins``
    each layer's saved U (or None).  ``dX`` and ``grads`` (one (dA, dB) per
    layer) optionally give the output buffers; they are overwritten.
    Returns (dX summed over the layers, [(dA, dB) per layer])."""
    import torch
    n = len(layers)
    if not 1 <= n <= 4 or len(dYs) != n:
        raise ValueError("one to four layers, one dY each")
    _matrix(X)
    T, d_in = X.shape[0], X.shape[1]
    r = 0 if layers[0][3] is None else layers[0][3].shape[0]
    tables = tables or [TABLE_NF4] * n
    U_ins = U_ins or [None] * n
    if grads is not None and len(grads) != n:
        raise ValueError("one (dA, dB) pair per layer")
    given, grads = grads, []
    descs = (Nf4Desc * n)()
    _check_in(X, (T, d_in), torch.bfloat16, "X")
    for i, (packed, codes, consts, A, B) in enumerate(layers):      # every layer's shapes first
        _check_weight(packed, codes, consts, f"layers[{i}]")
        if packed.shape[1] * 2 != d_in:
            raise ValueError(f"layers[{i}]: d_in {packed.shape[1] * 2} differs from X's {d_in}")
        _check_adapter(A, B, packed.shape[0], d_in, r, f"layers[{i}] ")
        _check_in(dYs[i], (T, packed.shape[0]), torch.bfloat16, f"dYs[{i}]")
    for i, (packed, codes, consts, A, B) in enumerate(layers):
        _need_cuda(packed, codes, consts, A, B, dYs[i], U_ins[i], name="qlora_linear_bwd_multi")
        _check_out(U_ins[i], (T, r), torch.float32, f"U_ins[{i}]")
        descs[i] = _stored_desc(packed, codes, consts, tables[i])
        if given is not None and r > 0:
            dA, dB = given[i]
            _check_out(dA, (r, d_in), torch.float32, f"grads[{i}] dA")
            _check_out(dB, (packed.shape[0], r), torch.float32, f"grads[{i}] dB")
            if dA is None or dB is None:
                raise ValueError(f"grads[{i}]: dA and dB are required")
            _need_cuda(dA, dB, name="qlora_linear_bwd_multi")
        else:
            dA = torch.empty((r, d_in), dtype=torch.float32, device=X.device) if r > 0 else None
            dB = torch.empty((packed.shape[0], r), dtype=torch.float32, device=X.device) if r > 0 else None
        grads.append((dA, dB))
    _need_cuda(X, dX, name="qlora_linear_bwd_multi")
    _check_out(dX, (T, d_in), torch.bfloat16, "dX")
    if dX is None and want_dx:
        dX = torch.empty((T, d_in), dtype=torch.bfloat16, device=X.device)
    n_b = ctypes.c_size_t()
    _check(lib().qlora_multi_bwd_workspace_bytes(n, descs, int(T), int(r), ctypes.byref(n_b)),
           "qlora_multi_bwd_workspace_bytes")
    ws = _workspace(n_b.value, X.device, workspace)
    arr = lambda vals: (ctypes.c_void_p * n)(*vals)
    _check(lib().qlora_linear_bwd_multi(
        n, descs, arr([_ptr(l[0]) for l in layers]), arr([_ptr(l[1]) for l in layers]),
        arr([_ptr(l[2]) for l in layers]), int(T), _ptr(X), int(r), float(alpha),
        arr([_ptr(l[3]) for l in layers]), arr([_ptr(l[4]) for l in layers]), arr([_ptr(u) for u in U_ins]),
        arr([_ptr(dy) for dy in dYs]), _ptr(dX), arr([_ptr(g[0]) for g in grads]), arr([_ptr(g[1]) for g in grads]),
        _ptr(ws), n_b.value, _stream(stream)), "qlora_linear_bwd_multi")
    return dX, grads


def qlora_linear_bwd(packed, codes, consts, X, A, B, alpha: float, dY, U_in=None, dX=None, dA=None, dB=None,
                     want_dx: bool = True, workspace=None, stream=None, table: int = TABLE_NF4,
                     accumulate: bool = False, keep=None, p: float = 0.0):
    """Backward: returns (dX bf16 [T][d_in] or None, dA fp32 [r][d_in], dB fp32 [d_out][r]).

    accumulate=True adds the adapter gradients to the given dA and dB
    (qlora_linear_bwd_accumulate) instead of overwriting them; keep / p as in
    qlora_linear_fwd (qlora_linear_bwd_dropout; pass the forward's U)."""
    import torch
    d_out, d_in = packed.shape[0], packed.shape[1] * 2
    _matrix(X)
    T = X.shape[0]
    r = 0 if A is None else A.shape[0]
    _check_weight(packed, codes, consts)
    _check_in(X, (T, d_in), torch.bfloat16, "X")
    _check_in(dY, (T, d_out), torch.bfloat16, "dY")
    _check_adapter(A, B, d_out, d_in, r)
    _need_cuda(packed, codes, consts, X, A, B, dY, U_in, dX, dA, dB, name="qlora_linear_bwd")
    _check_out(dX, (T, d_in), torch.bfloat16, "dX")
    _check_out(U_in, (T, r), torch.float32, "U_in")
    if dX is None and want_dx:
        dX = torch.empty((T, d_in), dtype=torch.bfloat16, device=X.device)
    if r > 0:
        if accumulate and (dA is None or dB is None):
            raise ValueError("accumulate=True needs the dA and dB to add to")
        if dA is None:
            dA = torch.empty((r, d_in), dtype=torch.float32, device=X.device)
        if dB is None:
            dB = torch.empty((d_out, r), dtype=torch.float32, device=X.device)
        for t, nm, shape in ((dA, "dA", (r, d_in)), (dB, "dB", (d_out, r))):
            if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError(f"{nm} must be a contiguous float32 tensor of shape {shape}")
    d = _stored_desc(packed, codes, consts, table)
    if keep is not None:
        _check_keep(keep, T, d_in)
        nbytes = _dropout_ws(d, T, r, 1)
        ws = _workspace(nbytes, X.device, workspace)
        _check(lib().qlora_linear_bwd_dropout(ctypes.byref(d), _ptr(packed), _ptr(codes), _ptr(consts), T, _ptr(X),
                                              r, float(alpha), _ptr(A), _ptr(B), _ptr(U_in), _ptr(dY), _ptr(keep),
                                              float(p), _ptr(dX), _ptr(dA), _ptr(dB), 1 if accumulate else 0,
                                              _ptr(ws), nbytes, _stream(stream)), "qlora_linear_bwd_dropout")
        return dX, dA, dB
    nbytes = qlora_bwd_workspace_bytes(d_out, d_in, T, r)
    ws = _workspace(nbytes, X.device, workspace)
    name = "qlora_linear_bwd_accumulate" if accumulate else "qlora_linear_bwd"
    _check(getattr(lib(), name)(ctypes.byref(d), _ptr(packed), _ptr(codes), _ptr(consts), T, _ptr(X), r,
                                float(alpha), _ptr(A), _ptr(B), _ptr(U_in), _ptr(dY), _ptr(dX), _ptr(dA),
                                _ptr(dB), _ptr(ws), nbytes, _stream(stream)), name)
    return dX, dA, dB


def qlora_dequantize_nf4(packed, codes, consts, W_hat=None, stream=None, table: int = TABLE_NF4):
    """Restored weight: bf16 [d_out][d_in], bit-identical to what the fused
    products restore on chip."""
    import torch
    d_out, d_in = packed.shape[0], packed.shape[1] * 2
    _check_weight(packed, codes, consts)
    _need_cuda(packed, codes, consts, W_hat, name="qlora_dequantize_nf4")
    _check_out(W_hat, (d_out, d_in), torch.bfloat16, "W_hat")
    if W_hat is None:
        W_hat = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=packed.device)
    d = _stored_desc(packed, codes, consts, table)
    _check(lib().qlora_dequantize_nf4(ctypes.byref(d), _ptr(packed), _ptr(codes), _ptr(consts), _ptr(W_hat),
                                      _stream(stream)), "qlora_dequantize_nf4")
    return W_hat


def qlora_merge_lora(packed, codes, consts, A, B, alpha: float, W_merged=None, stream=None,
                     table: int = TABLE_NF4):
    """The adapter merged into the restored weight: bf16 [d_out][d_in] =
    bf16(W_hat + (alpha / r) B A); A bf16 [r][d_in], B bf16 [d_out][r]."""
    import torch
    d_out, d_in = packed.shape[0], packed.shape[1] * 2
    r = A.shape[0]
    _check_weight(packed, codes, consts)
    if A is None or B is None:
        raise ValueError("A and B are required")
    _check_adapter(A, B, d_out, d_in, r)
    _need_cuda(packed, codes, consts, A, B, W_merged, name="qlora_merge_lora")
    _check_out(W_merged, (d_out, d_in), torch.bfloat16, "W_merged")
    if W_merged is None:
        W_merged = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=packed.device)
    d = _stored_desc(packed, codes, consts, table)
    _check(lib().qlora_merge_lora(ctypes.byref(d), _ptr(packed), _ptr(codes), _ptr(consts), int(r), float(alpha),
                                  _ptr(A), _ptr(B), _ptr(W_merged), _stream(stream)), "qlora_merge_lora")
    return W_merged


# ---------------------------------------------------------------------------
# Per-kernel timing (hipEvents recorded by the library around its launches)
# ---------------------------------------------------------------------------

def qlora_adamw_step(param, grad, exp_avg, exp_avg_sq, step: int, lr: float, betas=(0.9, 0.999),
                     eps: float = 1e-8, weight_decay: float = 0.0, grad_scale: float = 1.0, param_bf16=None,
                     stream=None):
    """AdamW update in place of fp32 param / exp_avg / exp_avg_sq (same size,
    contiguous, on the GPU) from fp32 grad; param_bf16 (bf16, same size) if
    given receives the rounded parameters.  Returns param_bf16."""
    import torch
    _need_cuda(param, grad, exp_avg, exp_avg_sq, param_bf16, name="qlora_adamw_step")
    n = param.numel()
    for t, nm in ((param, "param"), (grad, "grad"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous float32 tensor of {n} elements")
    if param_bf16 is not None and (param_bf16.dtype != torch.bfloat16 or param_bf16.numel() != n
                                   or not param_bf16.is_contiguous()):
        raise ValueError(f"param_bf16 must be a contiguous bfloat16 tensor of {n} elements")
    h = AdamwHparams(float(lr), float(betas[0]), float(betas[1]), float(eps), float(weight_decay),
                     float(grad_scale), int(step))
    _check(lib().qlora_adamw_step(ctypes.byref(h), n, _ptr(param), _ptr(grad), _ptr(exp_avg), _ptr(exp_avg_sq),
                                  _ptr(param_bf16), _stream(stream)), "qlora_adamw_step")
    return param_bf16


def qlora_trace_enable(enable: bool = True) -> None:
    _check(lib().qlora_trace_enable(1 if enable else 0), "qlora_trace_enable")


def qlora_trace_kernel_name(kernel: int):
    n = lib().qlora_trace_kernel_name(int(kernel))
    return None if n is None else n.decode()


def qlora_trace_select(names) -> None:
    """Bracket only the named kernels (names as reported by qlora_trace_read)."""
    mask = 0
    k = 0
    while True:
        n = qlora_trace_kernel_name(k)
        if n is None:
            break
        if n in names:
            mask |= 1 << k
        k += 1
    _check(lib().qlora_trace_select(mask), "qlora_trace_select")


def qlora_trace_read(reset: bool = True) -> dict:
    """{kernel name: (launches, total_ms)} for the launches recorded so far."""
    stats = (KernelStat * 32)()
    n = ctypes.c_int()
    _check(lib().qlora_trace_read(stats, 32, ctypes.byref(n), 1 if reset else 0), "qlora_trace_read")
    return {stats[i].name.decode(): (int(stats[i].launches), float(stats[i].total_ms))
            for i in range(min(n.value, 32))}
