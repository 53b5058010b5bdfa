"""Python binding of the MI355X left-lower TRSM library (libtrsm_amd.so).

Argument marshalling only: every step of the solve runs in the library's HIP
kernels.  The functions carry the names of the C ABI (include/trsm.h):

    trsm_lln(A, B, alpha=1.0, *, stream=None)                      -> B
    trsm_solve(A, B, alpha=1.0, *, side, uplo, trans, diag, stream=None) -> B
    trsm_lln_strided_batched(A, B, alpha=1.0, *, stream=None)      -> B
    trsm_lln_ex(A, B, alpha=1.0, ib=0, force_blocked=False, *, stream=None) -> B
    trsm_lln_noalloc(A, B, alpha=1.0, *, stream=None)              -> B
    trsm_lln_select_ib(dtype, m, n)                                -> int
    trsm_status_string(status)                                     -> str
    trsm_release_workspace()

A and B are torch tensors on the GPU in column-major storage: for an m x n
operand, stride(0) == 1 and stride(1) == ld >= m (``colmajor_empty`` makes
one).  Batched operands are (batch, m, n) with strides (stride, 1, ld).
Supported dtypes: torch.float32, torch.float64, torch.complex64,
torch.complex128.  B is overwritten with X such that L X = alpha B, L the
lower triangle of A (trsm_solve: the general op(A) X = alpha B or
X op(A) = alpha B).

The library must have been built (``python triangular_solve_trsm_amd/build.py``
or ``__graft_entry__.build()``); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtrsm_amd.so")

R32F, R64F, C64F, C32F = 0, 1, 2, 3
STATUS = {0: "SUCCESS", 1: "INVALID_VALUE", 2: "ALLOC_FAILED", 3: "HIP_ERROR", 4: "NOT_SUPPORTED"}
IB_CHOICES = (64, 128, 256, 512, 1024)

# Every symbol include/trsm.h and include/trsm_kernels.h declare.
EXPORTS = ("trsm_lln", "trsm_solve", "trsm_lln_strided_batched", "trsm_lln_ex", "trsm_lln_noalloc",
           "trsm_lln_select_ib",
           "trsm_status_string", "trsm_release_workspace",
           "trsm_kernel_diag_inv", "trsm_kernel_gemm",
           "trsm_profile_start", "trsm_profile_select", "trsm_profile_stop", "trsm_profile_count",
           "trsm_profile_read")

KERNEL_KINDS = {0: "small", 1: "diag_inv", 2: "copy", 3: "solve_gemm", 4: "update_gemm", 5: "fill"}


class ProfileRecord(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("m", ctypes.c_int64),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("batch", ctypes.c_int64),
                ("ms", ctypes.c_float)]


class TrsmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python triangular_solve_trsm_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.trsm_lln.argtypes = [ci, i64, i64, vp, vp, i64, vp, i64, vp]
    lib.trsm_lln.restype = ci
    lib.trsm_lln_strided_batched.argtypes = [ci, i64, i64, vp, vp, i64, i64, vp, i64, i64, i64, vp]
    lib.trsm_lln_strided_batched.restype = ci
    lib.trsm_lln_ex.argtypes = [ci, i64, i64, vp, vp, i64, vp, i64, ci, ci, vp]
    lib.trsm_lln_noalloc.argtypes = [ci, i64, i64, vp, vp, i64, vp, i64, vp]
    lib.trsm_lln_noalloc.restype = ci
    lib.trsm_solve.argtypes = [ci, ci, ci, ci, ci, i64, i64, vp, vp, i64, vp, i64, vp]
    lib.trsm_solve.restype = ci
    lib.trsm_lln_ex.restype = ci
    lib.trsm_lln_select_ib.argtypes = [ci, i64, i64]
    lib.trsm_lln_select_ib.restype = ci
    lib.trsm_status_string.argtypes = [ci]
    lib.trsm_status_string.restype = ctypes.c_char_p
    lib.trsm_release_workspace.argtypes = []
    lib.trsm_release_workspace.restype = ci
    lib.trsm_kernel_diag_inv.argtypes = [ci, ci, i64, vp, i64, vp, vp]
    lib.trsm_kernel_diag_inv.restype = ci
    lib.trsm_kernel_gemm.argtypes = [ci, i64, i64, i64, vp, vp, vp, i64, vp, i64, vp, i64,
                                     vp, i64, vp, i64, i64, ci, vp]
    lib.trsm_kernel_gemm.restype = ci
    lib.trsm_profile_start.argtypes = []
    lib.trsm_profile_start.restype = ci
    lib.trsm_profile_select.argtypes = [ctypes.c_uint32]
    lib.trsm_profile_select.restype = ci
    lib.trsm_profile_stop.argtypes = []
    lib.trsm_profile_stop.restype = ci
    lib.trsm_profile_count.argtypes = []
    lib.trsm_profile_count.restype = i64
    lib.trsm_profile_read.argtypes = [i64, ctypes.POINTER(ProfileRecord)]
    lib.trsm_profile_read.restype = ci
    return lib


lib = _load()


# ---- marshalling helpers ---------------------------------------------------

_DTYPE_CODES = None


def _dtype_code(t) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        _DTYPE_CODES = {torch.float32: R32F, torch.float64: R64F, torch.complex128: C64F,
                        torch.complex64: C32F}
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float64, complex64 or complex128")
    return code


def alpha_buffer(code: int, alpha):
    """Host scalar in the layout the ABI expects (float / double / double[2] /
    float[2])."""
    if code == R32F:
        return ctypes.c_float(float(alpha))
    if code == R64F:
        return ctypes.c_double(float(alpha))
    a = complex(alpha)
    if code == C32F:
        return (ctypes.c_float * 2)(a.real, a.imag)
    return (ctypes.c_double * 2)(a.real, a.imag)


_RAW_STREAM = None


def _stream_handle(stream, dev: int = None) -> int:
    """The stream argument of a call: the given torch stream (or raw handle),
    else torch's current stream, on device `dev` when the caller has already
    established it (its raw handle is read without building a Stream object,
    a few microseconds per call on a small solve)."""
    global _RAW_STREAM
    if stream is None:
        import torch
        if dev is not None:
            if _RAW_STREAM is None:
                _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", False)
            if _RAW_STREAM:
                return int(_RAW_STREAM(dev))
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ld(t, rows: int, cols: int) -> int:
    """Leading dimension of a column-major 2-D view (stride(-2) must be 1)."""
    if rows == 0 or cols == 0:
        return max(rows, 1)  # empty operand: its strides mean nothing
    s0, s1 = t.stride(-2), t.stride(-1)
    if rows > 1 and s0 != 1:
        raise ValueError("operand must be column-major: stride of the row index must be 1")
    ld = s1 if cols > 1 else max(rows, 1)
    return max(ld, 1)


def _check_device(where: str, *tensors, stream=None):
    """Every operand must be a tensor in GPU memory, all on one device, and
    an explicit torch stream must belong to that device: the library takes
    raw device pointers, and a host pointer reaching a kernel faults the GPU.
    Raises before anything is handed to the library.  Returns the device
    index (None when every operand is None)."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not getattr(t, "is_cuda", False):
            raise ValueError(f"{where}: every operand must be a GPU tensor "
                             f"(got one on {getattr(t, 'device', type(t).__name__)})")
        d = t.get_device()
        if dev is None:
            dev = d
        elif d != dev:
            raise ValueError(f"{where}: operands on different devices (cuda:{dev} and cuda:{d})")
    sdev = getattr(stream, "device", None)
    if dev is not None and sdev is not None and sdev.index != dev:
        raise ValueError(f"{where}: stream on {sdev} but operands on cuda:{dev}")
    if dev is not None:
        import torch
        cur = torch.cuda.current_device()
        if cur != dev:
            raise ValueError(f"{where}: operands on cuda:{dev} but the current device is "
                             f"cuda:{cur} (use torch.cuda.device)")
    return dev


def _check(status: int, where: str):
    if status != 0:
        raise TrsmError(status, where)


def colmajor_empty(m: int, n: int, ld: int = None, *, dtype=None, device="cuda", batch: int = None):
    """Uninitialised column-major tensor (m x n, leading dimension ld)."""
    import torch
    ld = max(m, 1) if ld is None else ld
    if batch is None:
        return torch.empty((n, ld), dtype=dtype, device=device).T[:m]
    return torch.empty((batch, n, ld), dtype=dtype, device=device).transpose(1, 2)[:, :m]


# ---- the ABI, by name -------------------------------------------------------

def trsm_lln(A, B, alpha=1.0, *, stream=None):
    """Solve L X = alpha B in place (B <- X); L is the lower triangle of A."""
    code = _dtype_code(B)
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    m, n = B.shape
    if tuple(A.shape) != (m, m):
        raise ValueError(f"A must be {m} x {m}")
    lda, ldb = _ld(A, m, m), _ld(B, m, n)
    dev = _check_device("trsm_lln", A, B, stream=stream)
    al = alpha_buffer(code, alpha)
    st = lib.trsm_lln(code, m, n, ctypes.addressof(al), A.data_ptr(), lda, B.data_ptr(), ldb,
                      _stream_handle(stream, dev))
    _check(st, "trsm_lln")
    return B


NOALLOC_MAX_WORKSPACE_BYTES = 128 << 20  # TRSM_NOALLOC_MAX_WORKSPACE_BYTES of trsm.h


def trsm_lln_noalloc(A, B, alpha=1.0, *, stream=None):
    """trsm_lln without any allocation: the blocked path's workspace is the
    library's fixed per-device scratch array (NOALLOC_MAX_WORKSPACE_BYTES);
    larger problems raise TrsmError (INVALID_VALUE) with B untouched.  Calls
    that may overlap in time on one device race on that array."""
    code = _dtype_code(B)
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    m, n = B.shape
    if tuple(A.shape) != (m, m):
        raise ValueError(f"A must be {m} x {m}")
    lda, ldb = _ld(A, m, m), _ld(B, m, n)
    dev = _check_device("trsm_lln_noalloc", A, B, stream=stream)
    al = alpha_buffer(code, alpha)
    st = lib.trsm_lln_noalloc(code, m, n, ctypes.addressof(al), A.data_ptr(), lda, B.data_ptr(), ldb,
                              _stream_handle(stream, dev))
    _check(st, "trsm_lln_noalloc")
    return B


def trsm_solve(A, B, alpha=1.0, *, side="L", uplo="L", trans="N", diag="N", stream=None):
    """General TRSM in place (B <- X): op(A) X = alpha B for side 'L' (A is
    m x m), X op(A) = alpha B for side 'R' (A is n x n); uplo 'L' / 'U' is the
    triangle of A used, trans 'N' / 'T' / 'C' gives op(A) = A, A^T, A^H, and
    diag 'U' means a unit diagonal that is not read."""
    code = _dtype_code(B)
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    m, n = B.shape
    k = m if side == "L" else n
    if tuple(A.shape) != (k, k):
        raise ValueError(f"A must be {k} x {k}")
    flags = ({"L": 0, "R": 1}[side], {"L": 0, "U": 1}[uplo], {"N": 0, "T": 1, "C": 2}[trans],
             {"N": 0, "U": 1}[diag])
    lda, ldb = _ld(A, k, k), _ld(B, m, n)
    dev = _check_device("trsm_solve", A, B, stream=stream)
    al = alpha_buffer(code, alpha)
    st = lib.trsm_solve(*flags, code, m, n, ctypes.addressof(al), A.data_ptr(), lda,
                        B.data_ptr(), ldb, _stream_handle(stream, dev))
    _check(st, "trsm_solve")
    return B


def trsm_lln_ex(A, B, alpha=1.0, ib: int = 0, force_blocked: bool = False, *, stream=None):
    """trsm_lln with a forced diagonal block size (0 = table) and optional
    use of the blocked path at m <= 64."""
    code = _dtype_code(B)
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    m, n = B.shape
    if tuple(A.shape) != (m, m):
        raise ValueError(f"A must be {m} x {m}")
    lda, ldb = _ld(A, m, m), _ld(B, m, n)
    dev = _check_device("trsm_lln_ex", A, B, stream=stream)
    al = alpha_buffer(code, alpha)
    st = lib.trsm_lln_ex(code, m, n, ctypes.addressof(al), A.data_ptr(), lda, B.data_ptr(), ldb,
                         int(ib), int(bool(force_blocked)), _stream_handle(stream, dev))
    _check(st, "trsm_lln_ex")
    return B


def trsm_lln_strided_batched(A, B, alpha=1.0, *, stream=None):
    """Batched solve: A (batch, m, m), B (batch, m, n), each problem
    column-major, problems at a constant element stride."""
    code = _dtype_code(B)
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    batch, m, n = B.shape
    if tuple(A.shape) != (batch, m, m):
        raise ValueError(f"A must be {batch} x {m} x {m}")
    lda, ldb = _ld(A, m, m), _ld(B, m, n)
    dev = _check_device("trsm_lln_strided_batched", A, B, stream=stream)
    al = alpha_buffer(code, alpha)
    st = lib.trsm_lln_strided_batched(code, m, n, ctypes.addressof(al), A.data_ptr(), lda,
                                      A.stride(0) if batch > 1 else 0, B.data_ptr(), ldb,
                                      B.stride(0) if batch > 1 else 0, batch, _stream_handle(stream, dev))
    _check(st, "trsm_lln_strided_batched")
    return B


def trsm_lln_select_ib(dtype, m: int, n: int) -> int:
    """Block size of the offline table for (dtype, m, n); dtype is a torch
    dtype or one of R32F / R64F / C64F / C32F."""
    if not isinstance(dtype, int):
        import torch
        dtype = {torch.float32: R32F, torch.float64: R64F, torch.complex128: C64F, torch.complex64: C32F}[dtype]
    return int(lib.trsm_lln_select_ib(dtype, m, n))


def trsm_status_string(status: int) -> str:
    return lib.trsm_status_string(int(status)).decode()


def trsm_release_workspace():
    _check(lib.trsm_release_workspace(), "trsm_release_workspace")


# ---- step-level entry points (include/trsm_kernels.h) -----------------------

def trsm_kernel_diag_inv(A, W, ib: int, *, stream=None):
    """Invert every ib x ib diagonal block of the lower triangle of A (m x m,
    column-major) into W (a contiguous buffer of ceil(m/ib)*ib*ib elements;
    block t at offset t*ib*ib, column-major, leading dimension ib)."""
    code = _dtype_code(A)
    m = A.shape[0]
    nb = (m + ib - 1) // ib
    if W.dtype != A.dtype or W.numel() < nb * ib * ib or not W.is_contiguous():
        raise ValueError("W must be a contiguous buffer of ceil(m/ib)*ib*ib elements of A's dtype")
    dev = _check_device("trsm_kernel_diag_inv", A, W, stream=stream)
    st = lib.trsm_kernel_diag_inv(code, int(ib), m, A.data_ptr(), _ld(A, m, m), W.data_ptr(),
                                  _stream_handle(stream, dev))
    _check(st, "trsm_kernel_diag_inv")
    return W


def trsm_kernel_gemm(A, Bm, D, *, beta=0.0, gamma=1.0, C=None, D2=None, split: int = 0,
                     a_lower: bool = False, stream=None):
    """D = beta*C + gamma*(A @ Bm) on the MFMA GEMM of the blocked path; rows
    [0, split) go to D2 when given.  All operands column-major."""
    code = _dtype_code(D)
    M, K = A.shape
    K2, N = Bm.shape
    if K2 != K or tuple(D.shape) != (M, N):
        raise ValueError("shape mismatch")
    dev = _check_device("trsm_kernel_gemm", A, Bm, D, C, D2, stream=stream)
    b = alpha_buffer(code, beta)
    g = alpha_buffer(code, gamma)
    c_ptr = C.data_ptr() if C is not None else None
    ldc = _ld(C, M, N) if C is not None else max(M, 1)
    d2_ptr = D2.data_ptr() if D2 is not None else None
    ldd2 = _ld(D2, D2.shape[0], N) if D2 is not None else max(M, 1)
    st = lib.trsm_kernel_gemm(code, M, N, K, ctypes.addressof(b), ctypes.addressof(g),
                              A.data_ptr(), _ld(A, M, K), Bm.data_ptr(), _ld(Bm, K, N),
                              c_ptr, ldc, D.data_ptr(), _ld(D, M, N), d2_ptr, ldd2,
                              int(split), int(bool(a_lower)), _stream_handle(stream, dev))
    _check(st, "trsm_kernel_gemm")
    return D


def trsm_profile_start():
    _check(lib.trsm_profile_start(), "trsm_profile_start")


def trsm_profile_select(kinds=None):
    """Record only launches of the given kinds (names of KERNEL_KINDS, or
    None for every kind)."""
    if kinds is None:
        mask = 0xFFFFFFFF
    else:
        codes = {v: k for k, v in KERNEL_KINDS.items()}
        mask = 0
        for k in kinds:
            mask |= 1 << codes[k]
    _check(lib.trsm_profile_select(mask), "trsm_profile_select")


def trsm_profile_stop():
    _check(lib.trsm_profile_stop(), "trsm_profile_stop")


def trsm_profile_count() -> int:
    return int(lib.trsm_profile_count())


def trsm_profile_read(i: int) -> dict:
    rec = ProfileRecord()
    _check(lib.trsm_profile_read(int(i), ctypes.byref(rec)), "trsm_profile_read")
    return {"kind": KERNEL_KINDS.get(rec.kind, rec.kind), "dtype": rec.dtype, "m": rec.m,
            "n": rec.n, "k": rec.k, "batch": rec.batch, "ms": float(rec.ms)}


def profile_records() -> list:
    """All records of the current profile (waits for their launches)."""
    return [trsm_profile_read(i) for i in range(trsm_profile_count())]
