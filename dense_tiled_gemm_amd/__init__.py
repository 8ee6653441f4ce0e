"""Python binding of libgemm_bt.so: C = A·Bᵀ on an MI355X (gfx950).

Argument marshalling only.  Every arithmetic step runs in the library's HIP
kernels; PyTorch supplies device memory and the stream.  There is no CPU or
PyTorch fallback: if the shared library is missing, every call raises.

Entry points (same names as the C-ABI in ``include/gemm_bt.h``):
  gemm_bt(A, B, C, M, N, K, in_dtype, out_dtype, stream)   raw device pointers
  gemm_bt_batched(A, B, C, batch, M, N, K, stride_a, stride_b, stride_c, in_dtype, out_dtype, stream)
  gemm_bt_layout(A, B, C, M, N, K, a_layout, b_layout, in_dtype, out_dtype, stream)
  gemm_bt_batched_layout(A, B, C, batch, M, N, K, stride_a, stride_b, stride_c, a_layout, b_layout, in_dtype,
                         out_dtype, stream)
  gemm_bt_status_string(status), gemm_bt_version()
  gemm_bt_plan(M, N, K, in_dtype, out_dtype, a_align, b_align, c_align)
  gemm_bt_plan_batched(batch, M, N, K, in_dtype, out_dtype, a_align, b_align, c_align)
  gemm_bt_plan_layout(M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_align, b_align, c_align)
  gemm_bt_plan_batched_layout(batch, M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_align, b_align, c_align)
  gemm_bt_tile_coord(pid, tiles_m, tiles_n, group_m)
  gemm_bt_ws(A, B, C, M, N, K, in_dtype, out_dtype, workspace, workspace_bytes, stream)   stream-K
  gemm_bt_workspace_size(M, N, K, in_dtype, out_dtype), gemm_bt_plan_ws(M, N, K, in_dtype, out_dtype, ...)
  gemm_bt_noalloc(A, B, C, M, N, K, in_dtype, out_dtype, stream)   gemm_bt_ws with the library's scratch
and torch convenience wrappers ``mm_bt(a, b, out_dtype)`` (2-D or batched 3-D operands),
``mm_layout(a, b, a_layout, b_layout, out_dtype)`` and ``mm(a, b, out_dtype)`` (= a @ b).
"""
from __future__ import annotations

import ctypes
import os
import threading

F32, F16, BF16, FP8_E4M3, FP8_E5M2, INT8, INT32 = 0, 1, 2, 3, 4, 5, 6
OK, ERR_INVALID_VALUE, ERR_UNSUPPORTED, ERR_NO_DEVICE, ERR_LAUNCH = 0, 1, 2, 3, 4
K_INNER, K_OUTER = 0, 1  # operand layouts of gemm_bt_layout

_HERE = os.path.dirname(os.path.abspath(__file__))
# GEMM_BT_LIB may name another build of this library (e.g. a build with the tuning variants, for measurements)
LIB_PATH = os.environ.get("GEMM_BT_LIB") or os.path.join(_HERE, "libgemm_bt.so")
EXPORTS = ("gemm_bt", "gemm_bt_batched", "gemm_bt_layout", "gemm_bt_batched_layout", "gemm_bt_status_string",
           "gemm_bt_version", "gemm_bt_plan", "gemm_bt_plan_batched", "gemm_bt_plan_layout",
           "gemm_bt_plan_batched_layout", "gemm_bt_tile_coord", "gemm_bt_ws", "gemm_bt_workspace_size",
           "gemm_bt_plan_ws", "gemm_bt_noalloc")
SK_COUNTER_BYTES = 16384  # leading counter area of a gemm_bt_ws workspace (zero between calls)

_lock = threading.Lock()
_lib = None


class GemmBtError(RuntimeError):
    def __init__(self, status, what="gemm_bt"):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("variant", ctypes.c_int), ("bm", ctypes.c_int), ("bn", ctypes.c_int),
                ("bk", ctypes.c_int), ("threads", ctypes.c_int), ("vec", ctypes.c_int), ("group_m", ctypes.c_int),
                ("ksplit", ctypes.c_int), ("stages", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("tiles_m", ctypes.c_int64),
                ("tiles_n", ctypes.c_int64), ("grid", ctypes.c_int64), ("batch", ctypes.c_int64),
                ("split_tiles", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64), ("split_rows", ctypes.c_int64),
                ("split_items", ctypes.c_int64)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def load():
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:  # fast path for the raw calls below, made once per launch
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libgemm_bt.so is not built (expected at %s); run "
                                   "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            lib.gemm_bt.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
            lib.gemm_bt.restype = ci
            lib.gemm_bt_batched.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, ci, vp]
            lib.gemm_bt_batched.restype = ci
            lib.gemm_bt_plan_batched.argtypes = [i64, i64, i64, i64, ci, ci, ci, ci, ci, ctypes.POINTER(Plan)]
            lib.gemm_bt_plan_batched.restype = ci
            lib.gemm_bt_layout.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ci, ci, vp]
            lib.gemm_bt_layout.restype = ci
            lib.gemm_bt_plan_layout.argtypes = [i64, i64, i64, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(Plan)]
            lib.gemm_bt_plan_layout.restype = ci
            lib.gemm_bt_batched_layout.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, ci, ci, ci, vp]
            lib.gemm_bt_batched_layout.restype = ci
            lib.gemm_bt_plan_batched_layout.argtypes = [i64, i64, i64, i64, ci, ci, ci, ci, ci, ci, ci,
                                                        ctypes.POINTER(Plan)]
            lib.gemm_bt_plan_batched_layout.restype = ci
            lib.gemm_bt_status_string.argtypes = [ci]
            lib.gemm_bt_status_string.restype = ctypes.c_char_p
            lib.gemm_bt_version.argtypes = []
            lib.gemm_bt_version.restype = ci
            lib.gemm_bt_plan.argtypes = [i64, i64, i64, ci, ci, ci, ci, ci, ctypes.POINTER(Plan)]
            lib.gemm_bt_plan.restype = ci
            lib.gemm_bt_tile_coord.argtypes = [i64, i64, i64, ci, ctypes.POINTER(i64), ctypes.POINTER(i64)]
            lib.gemm_bt_tile_coord.restype = ci
            lib.gemm_bt_ws.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp, ctypes.c_size_t, vp]
            lib.gemm_bt_ws.restype = ci
            lib.gemm_bt_workspace_size.argtypes = [i64, i64, i64, ci, ci, ctypes.POINTER(ctypes.c_size_t)]
            lib.gemm_bt_workspace_size.restype = ci
            lib.gemm_bt_plan_ws.argtypes = [i64, i64, i64, ci, ci, ci, ci, ci, ctypes.POINTER(Plan)]
            lib.gemm_bt_plan_ws.restype = ci
            lib.gemm_bt_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
            lib.gemm_bt_noalloc.restype = ci
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().gemm_bt_status_string(int(status)).decode()


gemm_bt_status_string = status_string


def gemm_bt_version() -> int:
    return int(load().gemm_bt_version())


def gemm_bt(A: int, B: int, C: int, M: int, N: int, K: int, in_dtype: int, out_dtype: int,
            stream: int | None) -> int:
    """Raw call: device pointers as integers, returns the status code."""
    return int(load().gemm_bt(A or None, B or None, C or None, M, N, K, in_dtype, out_dtype, stream or None))


def gemm_bt_batched(A: int, B: int, C: int, batch: int, M: int, N: int, K: int, stride_a: int, stride_b: int,
                    stride_c: int, in_dtype: int, out_dtype: int, stream: int | None) -> int:
    """Raw batched call: item z uses A + z*stride_a etc. (strides in elements); returns the status code."""
    return int(load().gemm_bt_batched(A or None, B or None, C or None, batch, M, N, K, stride_a, stride_b, stride_c,
                                      in_dtype, out_dtype, stream or None))


def gemm_bt_layout(A: int, B: int, C: int, M: int, N: int, K: int, a_layout: int, b_layout: int, in_dtype: int,
                   out_dtype: int, stream: int | None) -> int:
    """Raw call with operand layouts (K_INNER / K_OUTER); returns the status code."""
    return int(load().gemm_bt_layout(A or None, B or None, C or None, M, N, K, a_layout, b_layout, in_dtype, out_dtype,
                                     stream or None))


def gemm_bt_plan_layout(M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_align=256, b_align=256, c_align=256):
    p = Plan()
    st = load().gemm_bt_plan_layout(M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_align, b_align, c_align,
                                    ctypes.byref(p))
    if st != OK:
        raise GemmBtError(st, "gemm_bt_plan_layout")
    return p


def gemm_bt_batched_layout(A: int, B: int, C: int, batch: int, M: int, N: int, K: int, stride_a: int, stride_b: int,
                           stride_c: int, a_layout: int, b_layout: int, in_dtype: int, out_dtype: int,
                           stream: int | None) -> int:
    """Raw batched call with operand layouts; returns the status code."""
    return int(load().gemm_bt_batched_layout(A or None, B or None, C or None, batch, M, N, K, stride_a, stride_b,
                                             stride_c, a_layout, b_layout, in_dtype, out_dtype, stream or None))


def gemm_bt_plan_batched_layout(batch, M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_align=256, b_align=256,
                                c_align=256):
    p = Plan()
    st = load().gemm_bt_plan_batched_layout(batch, M, N, K, a_layout, b_layout, in_dtype, out_dtype, a_align, b_align,
                                            c_align, ctypes.byref(p))
    if st != OK:
        raise GemmBtError(st, "gemm_bt_plan_batched_layout")
    return p


def gemm_bt_plan_batched(batch, M, N, K, in_dtype, out_dtype, a_align=256, b_align=256, c_align=256):
    p = Plan()
    st = load().gemm_bt_plan_batched(batch, M, N, K, in_dtype, out_dtype, a_align, b_align, c_align, ctypes.byref(p))
    if st != OK:
        raise GemmBtError(st, "gemm_bt_plan_batched")
    return p


def gemm_bt_plan(M, N, K, in_dtype, out_dtype, a_align=256, b_align=256, c_align=256):
    p = Plan()
    st = load().gemm_bt_plan(M, N, K, in_dtype, out_dtype, a_align, b_align, c_align, ctypes.byref(p))
    if st != OK:
        raise GemmBtError(st, "gemm_bt_plan")
    return p


def gemm_bt_ws(A: int, B: int, C: int, M: int, N: int, K: int, in_dtype: int, out_dtype: int, workspace: int,
               workspace_bytes: int, stream: int | None) -> int:
    """Raw stream-K call with a caller workspace (device pointer, bytes); returns the status code."""
    return int(load().gemm_bt_ws(A or None, B or None, C or None, M, N, K, in_dtype, out_dtype, workspace or None,
                                 workspace_bytes, stream or None))


def gemm_bt_noalloc(A: int, B: int, C: int, M: int, N: int, K: int, in_dtype: int, out_dtype: int,
                    stream: int | None) -> int:
    """Raw call of gemm_bt_ws with the library's own scratch (allocates nothing); returns the status code."""
    return int(load().gemm_bt_noalloc(A or None, B or None, C or None, M, N, K, in_dtype, out_dtype, stream or None))


def gemm_bt_workspace_size(M, N, K, in_dtype, out_dtype) -> int:
    n = ctypes.c_size_t()
    st = load().gemm_bt_workspace_size(M, N, K, in_dtype, out_dtype, ctypes.byref(n))
    if st != OK:
        raise GemmBtError(st, "gemm_bt_workspace_size")
    return n.value


def gemm_bt_plan_ws(M, N, K, in_dtype, out_dtype, a_align=256, b_align=256, c_align=256):
    p = Plan()
    st = load().gemm_bt_plan_ws(M, N, K, in_dtype, out_dtype, a_align, b_align, c_align, ctypes.byref(p))
    if st != OK:
        raise GemmBtError(st, "gemm_bt_plan_ws")
    return p


def gemm_bt_tile_coord(pid, tiles_m, tiles_n, group_m):
    tm, tn = ctypes.c_int64(), ctypes.c_int64()
    st = load().gemm_bt_tile_coord(pid, tiles_m, tiles_n, group_m, ctypes.byref(tm), ctypes.byref(tn))
    if st != OK:
        raise GemmBtError(st, "gemm_bt_tile_coord")
    return tm.value, tn.value


# ---------------------------------------------------------------- torch convenience

def _torch_code(dt):
    import torch

    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float16:
        return F16
    if dt == torch.float32:
        return F32
    if dt == torch.float8_e4m3fn:
        return FP8_E4M3
    if dt == torch.float8_e5m2:
        return FP8_E5M2
    if dt == torch.int8:
        return INT8
    if dt == torch.int32:
        return INT32
    raise TypeError("unsupported dtype %s" % dt)


def _torch_dtype(code):
    import torch

    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16, INT32: torch.int32}[code]


def _batch_operand(x):
    """(tensor, item stride in elements) of a 2-D or 3-D operand: a 2-D operand, or a 3-D one whose batch
    stride is 0 over contiguous items (``expand``), is shared by every item; others are made contiguous."""
    if x.dim() == 2:
        return x.contiguous(), 0
    if x.shape[0] > 0 and x.stride(0) == 0 and x[0].is_contiguous():
        return x[0], 0
    x = x.contiguous()
    return x, x.shape[1] * x.shape[2]


_ws_lock = threading.Lock()
_ws_cache = {}


def workspace_for(device, stream: int, nbytes: int):
    """A zero-initialised uint8 device tensor of at least `nbytes` for gemm_bt_ws calls on `stream`, kept per
    (device, stream) and reused: calls on one stream run in order, and each call leaves the counter area zero
    again.  Grows (a new zeroed tensor) when a larger size is asked for."""
    import torch

    key = (torch.device(device).index, int(stream))
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is None or ws.numel() < nbytes:
            with torch.cuda.device(device):
                ws = torch.zeros(max(nbytes, SK_COUNTER_BYTES), dtype=torch.uint8, device=device)
            _ws_cache[key] = ws
        return ws


def mm_bt(a, b, out_dtype=None, out=None, stream=None, split_k=True):
    """C = a @ b.T for CUDA/HIP tensors a (M×K) and b (N×K) of one input dtype.

    Batched: a (Z×M×K) and/or b (Z×N×K) give C (Z×M×N), C[z] = a[z] @ b[z].T;
    a 2-D operand (or one expanded along the batch) is shared by every item.
    Inputs: bfloat16, float16, float8_e4m3fn, float8_e5m2 or int8 (8-bit
    inputs need K % 16 == 0; int8 also K <= 131071).  ``out_dtype`` defaults
    to a's dtype (bfloat16 for 8-bit float inputs, which are not an output
    format; int32, the only one allowed, for int8); ``out`` may be a preallocated
    contiguous M×N (Z×M×N) tensor.  The call is asynchronous on ``stream``
    (default: torch's current stream of a's device).  With ``split_k`` (the
    default) a single product goes through gemm_bt_ws with a workspace kept
    per stream (``workspace_for``), so shapes whose tiles leave compute units
    idle are split along K (stream-K); ``split_k=False`` calls gemm_bt.
    """
    import torch

    if a.dim() not in (2, 3) or b.dim() not in (2, 3) or a.shape[-1] != b.shape[-1]:
        raise ValueError("expected a (M,K) or (Z,M,K) and b (N,K) or (Z,N,K), got %s and %s"
                         % (tuple(a.shape), tuple(b.shape)))
    if a.dim() == 3 and b.dim() == 3 and a.shape[0] != b.shape[0]:
        raise ValueError("batch sizes differ: %d and %d" % (a.shape[0], b.shape[0]))
    if a.dtype != b.dtype:
        raise TypeError("a and b must share one dtype")
    if not a.is_cuda or not b.is_cuda or a.device != b.device:
        raise ValueError("a and b must be on the same GPU")
    in_code = _torch_code(a.dtype)
    default_out = BF16 if in_code in (FP8_E4M3, FP8_E5M2) else (INT32 if in_code == INT8 else in_code)
    out_code = default_out if out_dtype is None else (_torch_code(out_dtype) if not isinstance(out_dtype, int)
                                                      else out_dtype)
    batched = a.dim() == 3 or b.dim() == 3
    Z = a.shape[0] if a.dim() == 3 else (b.shape[0] if b.dim() == 3 else 1)
    M, K = a.shape[-2], a.shape[-1]
    N = b.shape[-2]
    a, sa = _batch_operand(a)
    b, sb = _batch_operand(b)
    shape = (Z, M, N) if batched else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=_torch_dtype(out_code), device=a.device)
    elif tuple(out.shape) != shape or not out.is_contiguous() or out.dtype != _torch_dtype(out_code):
        raise ValueError("out must be a contiguous %s %s tensor" % ("x".join(map(str, shape)), _torch_dtype(out_code)))
    if stream is None:
        stream = torch.cuda.current_stream(a.device).cuda_stream
    with torch.cuda.device(a.device):
        if batched:
            st = gemm_bt_batched(a.data_ptr(), b.data_ptr(), out.data_ptr(), Z, M, N, K, sa, sb, M * N, in_code,
                                 out_code, stream)
        else:
            nbytes = gemm_bt_workspace_size(M, N, K, in_code, out_code) if split_k else 0
            if nbytes:
                ws = workspace_for(a.device, stream, nbytes)
                st = gemm_bt_ws(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, in_code, out_code,
                                ws.data_ptr(), ws.numel(), stream)
            else:
                st = gemm_bt(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, in_code, out_code, stream)
    if st != OK:
        raise GemmBtError(st)
    return out


def mm_layout(a, b, a_layout=K_INNER, b_layout=K_INNER, out_dtype=None, out=None, stream=None):
    """C = op(a) @ op(b).T for 16-bit tensors: a is (M,K) for K_INNER or (K,M) for K_OUTER, b is (N,K) for
    K_INNER or (K,N) for K_OUTER.  Either may carry a leading batch dimension Z (then C is (Z,M,N)); a 2-D
    operand, or one expanded along the batch, is shared by every item.  Operands stored K-outer are
    transposed inside the kernel."""
    import torch

    if a.dim() not in (2, 3) or b.dim() not in (2, 3):
        raise ValueError("expected 2-D or 3-D operands")
    if a.dim() == 3 and b.dim() == 3 and a.shape[0] != b.shape[0]:
        raise ValueError("batch sizes differ: %d and %d" % (a.shape[0], b.shape[0]))
    M, K = (a.shape[-1], a.shape[-2]) if a_layout == K_OUTER else (a.shape[-2], a.shape[-1])
    N, Kb = (b.shape[-1], b.shape[-2]) if b_layout == K_OUTER else (b.shape[-2], b.shape[-1])
    if K != Kb:
        raise ValueError("inner dimensions differ: %d and %d" % (K, Kb))
    if a.dtype != b.dtype:
        raise TypeError("a and b must share one dtype")
    if not a.is_cuda or not b.is_cuda or a.device != b.device:
        raise ValueError("a and b must be on the same GPU")
    in_code = _torch_code(a.dtype)
    out_code = in_code if out_dtype is None else (_torch_code(out_dtype) if not isinstance(out_dtype, int)
                                                  else out_dtype)
    batched = a.dim() == 3 or b.dim() == 3
    Z = a.shape[0] if a.dim() == 3 else (b.shape[0] if b.dim() == 3 else 1)
    a, sa = _batch_operand(a)
    b, sb = _batch_operand(b)
    shape = (Z, M, N) if batched else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=_torch_dtype(out_code), device=a.device)
    elif tuple(out.shape) != shape or not out.is_contiguous() or out.dtype != _torch_dtype(out_code):
        raise ValueError("out must be a contiguous %s %s tensor" % ("x".join(map(str, shape)), _torch_dtype(out_code)))
    if stream is None:
        stream = torch.cuda.current_stream(a.device).cuda_stream
    with torch.cuda.device(a.device):
        st = gemm_bt_batched_layout(a.data_ptr(), b.data_ptr(), out.data_ptr(), Z, M, N, K, sa, sb, M * N, a_layout,
                                    b_layout, in_code, out_code, stream)
    if st != OK:
        raise GemmBtError(st)
    return out


def mm(a, b, out_dtype=None, out=None, stream=None):
    """C = a @ b for 16-bit tensors a (M,K) and b (K,N), or batches of them (Z,M,K) and (Z,K,N): B is read
    K-outer, as it lies in memory."""
    return mm_layout(a, b, K_INNER, K_OUTER, out_dtype, out, stream)
