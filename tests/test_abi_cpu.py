"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/trsm.h declares, rejects bad arguments before any HIP call, and takes
the quick returns (m == 0, n == 0, batch == 0) without touching the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def header_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(trsm_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def T():
    import triangular_solve_trsm_amd as T
    return T


def test_header_declares_expected_entry_points(T):
    assert header_functions() == sorted(T.EXPORTS)


def test_library_exports_every_declared_symbol(T):
    for name in header_functions():
        assert hasattr(T.lib, name), name
    # and they are real dynamic symbols of the shared object
    lib = ctypes.CDLL(T.LIB_PATH)
    for name in header_functions():
        getattr(lib, name)


def test_status_strings(T):
    for code, text in [(0, "success"), (1, "invalid value"), (2, "workspace allocation failed"),
                       (3, "HIP runtime error"), (4, "not supported"), (99, "unknown status")]:
        assert T.trsm_status_string(code) == text


def test_select_ib_table(T):
    for dt in (T.R32F, T.R64F, T.C64F):
        for m in (1, 65, 500, 1000, 4096, 8192, 100000):
            assert T.trsm_lln_select_ib(dt, m, m) in T.IB_CHOICES
    assert T.trsm_lln_select_ib(7, 100, 100) == 0
    assert T.trsm_lln_select_ib(T.R64F, -1, 5) == 0


FAKE = 0x1000  # never dereferenced: every call below returns before any HIP call


def call(T, dtype=1, m=4, n=3, alpha=1.0, A=FAKE, lda=4, B=FAKE, ldb=4):
    al = T.alpha_buffer(dtype if dtype in (0, 1, 2, 3) else 1, alpha)
    return T.lib.trsm_lln(dtype, m, n, ctypes.addressof(al), A, lda, B, ldb, None)


@pytest.mark.parametrize("kw", [
    dict(dtype=4), dict(dtype=-1), dict(m=-1), dict(n=-2), dict(lda=3), dict(ldb=3),
    dict(m=0, lda=0), dict(A=None), dict(B=None), dict(m=5, lda=4, ldb=5), dict(m=5, lda=5, ldb=4),
])
def test_invalid_arguments(T, kw):
    assert call(T, **kw) == 1


def test_null_alpha_invalid(T):
    assert T.lib.trsm_lln(1, 4, 3, None, FAKE, 4, FAKE, 4, None) == 1


@pytest.mark.parametrize("kw", [dict(m=0, lda=1, ldb=1), dict(n=0), dict(m=0, n=0, lda=1, ldb=1)])
def test_quick_return_without_device(T, kw):
    # null pointers are allowed when m*n == 0
    kw2 = dict(kw, A=None, B=None)
    assert call(T, **kw2) == 0


def test_batched_argument_checks(T):
    al = T.alpha_buffer(1, 1.0)
    f = T.lib.trsm_lln_strided_batched
    a = ctypes.addressof(al)
    assert f(1, 4, 3, a, FAKE, 4, 16, FAKE, 4, 12, -1, None) == 1      # batch < 0
    assert f(1, 4, 3, a, FAKE, 4, -16, FAKE, 4, 12, 2, None) == 1      # negative stride
    assert f(1, 4, 3, a, FAKE, 3, 16, FAKE, 4, 12, 2, None) == 1       # lda < m
    assert f(1, 4, 3, a, FAKE, 4, 16, FAKE, 4, 12, 0, None) == 0       # batch == 0
    assert f(1, 0, 3, a, None, 1, 0, None, 1, 0, 5, None) == 0         # m == 0


def test_ex_rejects_bad_block_size(T):
    al = T.alpha_buffer(1, 1.0)
    a = ctypes.addressof(al)
    for ib in (1, 32, 100, 2048, 768, -64):
        assert T.lib.trsm_lln_ex(1, 100, 3, a, FAKE, 100, FAKE, 100, ib, 0, None) == 1
    # valid block size, quick return
    assert T.lib.trsm_lln_ex(1, 100, 0, a, FAKE, 100, FAKE, 100, 128, 0, None) == 0


def test_python_binding_rejects_bad_layouts(T):
    import torch
    A = torch.zeros(4, 4, dtype=torch.float64)
    B = torch.zeros(4, 3, dtype=torch.float64)       # row-major: stride(0) != 1
    with pytest.raises(ValueError, match="column-major"):
        T.trsm_lln(A.T, B, 1.0)
    with pytest.raises(TypeError):
        T.trsm_lln(A.T, torch.zeros(3, 4, dtype=torch.int32).T, 1.0)
    with pytest.raises(ValueError):
        T.trsm_lln(torch.zeros(5, 5, dtype=torch.float64).T, torch.zeros(3, 4, dtype=torch.float64).T)


def test_kernel_entry_points_reject_bad_arguments(T):
    one = T.alpha_buffer(1, 1.0)
    zero = T.alpha_buffer(1, 0.0)
    a1, a0 = ctypes.addressof(one), ctypes.addressof(zero)
    f = T.lib.trsm_kernel_diag_inv
    assert f(1, 100, 10, FAKE, 10, FAKE, None) == 1       # ib not a candidate
    assert f(1, 64, 10, FAKE, 9, FAKE, None) == 1         # lda < m
    assert f(9, 64, 10, FAKE, 10, FAKE, None) == 1        # dtype
    assert f(1, 64, 0, None, 1, None, None) == 0          # m == 0
    g = T.lib.trsm_kernel_gemm
    #         dt M  N  K  beta gamma A    lda B    ldb C    ldc D    ldd D2   ldd2 split low
    assert g(1, 8, 4, 6, a0, a1, FAKE, 7, FAKE, 6, None, 8, FAKE, 8, None, 8, 0, 0, None) == 1  # lda < M
    assert g(1, 8, 4, 6, a0, a1, FAKE, 8, FAKE, 5, None, 8, FAKE, 8, None, 8, 0, 0, None) == 1  # ldb < K
    assert g(1, 8, 4, 6, a1, a1, FAKE, 8, FAKE, 6, None, 8, FAKE, 8, None, 8, 0, 0, None) == 1  # beta != 0, C null
    assert g(1, 8, 4, 6, a0, a1, FAKE, 8, FAKE, 6, None, 8, FAKE, 8, None, 8, 0, 1, None) == 1  # a_lower, M != K
    assert g(1, 8, 4, 8, a0, a1, FAKE, 8, FAKE, 8, None, 8, FAKE, 8, FAKE, 8, 9, 0, None) == 1  # split > M
    assert g(1, 8, 4, 8, a0, a1, FAKE, 8, FAKE, 8, None, 8, FAKE, 8, FAKE, 3, 4, 0, None) == 1  # ldd2 < split
    assert g(1, 0, 4, 8, a0, a1, None, 1, FAKE, 8, None, 1, None, 1, None, 1, 0, 0, None) == 0  # M == 0


def test_profiler_bookkeeping_without_launches(T):
    T.trsm_profile_select(["update_gemm", "small"])
    T.trsm_profile_select(None)
    with pytest.raises(KeyError):
        T.trsm_profile_select(["no_such_kind"])
    T.trsm_profile_start()
    assert T.trsm_profile_count() == 0
    T.trsm_profile_stop()
    with pytest.raises(T.TrsmError):
        T.trsm_profile_read(0)


@pytest.mark.parametrize("flags,dims", [
    ((2, 0, 0, 0), (4, 3, 4, 4)), ((0, 2, 0, 0), (4, 3, 4, 4)), ((0, 0, 3, 0), (4, 3, 4, 4)),
    ((0, 0, 0, 2), (4, 3, 4, 4)), ((-1, 0, 0, 0), (4, 3, 4, 4)),
    ((1, 0, 0, 0), (4, 6, 5, 4)),   # right side: A is n x n, lda < n
    ((0, 1, 1, 1), (4, 3, 3, 4)),   # left side: lda < m
    ((1, 1, 2, 0), (4, 3, 3, 3)),   # ldb < m
])
def test_general_solve_rejects_bad_arguments(T, flags, dims):
    m, n, lda, ldb = dims
    al = T.alpha_buffer(1, 1.0)
    assert T.lib.trsm_solve(*flags, 1, m, n, ctypes.addressof(al), FAKE, lda, FAKE, ldb, None) == 1


def test_general_solve_quick_returns(T):
    al = T.alpha_buffer(1, 1.0)
    a = ctypes.addressof(al)
    for side in (0, 1):
        assert T.lib.trsm_solve(side, 1, 2, 1, 1, 0, 5, a, None, 5, None, 1, None) == 0   # m == 0
        assert T.lib.trsm_solve(side, 1, 2, 1, 1, 5, 0, a, None, 5, None, 5, None) == 0   # n == 0
    assert T.lib.trsm_solve(0, 0, 0, 0, 9, 4, 3, a, FAKE, 4, FAKE, 4, None) == 1         # dtype


def _table():
    """(dtype code, m, n) -> (ib, left) from the committed block-size table."""
    import re
    here = os.path.dirname(os.path.abspath(__file__))
    src = open(os.path.join(here, "..", "triangular_solve_trsm_amd", "csrc", "ib_table.inc")).read()
    codes = {"R32F": 0, "R64F": 1, "C64F": 2, "C32F": 3}
    out = {}
    for dt, m, n, ib, left in re.findall(r"\{(R32F|R64F|C64F|C32F), (\d+), (\d+), (\d+), ([01])\}", src):
        out[(codes[dt], int(m), int(n))] = (int(ib), int(left))
    return out


def test_block_size_lookup_matches_table(T):
    """Online lookup of section 4.3.2: at every profiled (m, n) the library
    returns that entry's block size; between entries it returns the entry
    nearest in log distance |log2(m/m_e)| + |log2(n/n_e)|."""
    import math
    table = _table()
    assert len(table) >= 4 * 20, "table should cover four types at many (m, n)"
    for (dt, m, n), (ib, _) in table.items():
        assert T.trsm_lln_select_ib(dt, m, n) == ib, (dt, m, n)
    for dt in range(4):
        entries = [(m, n, v[0]) for (d, m, n), v in table.items() if d == dt]
        for m, n in [(100, 100), (3000, 3000), (3000, 100), (6000, 300), (20000, 50), (700, 5000)]:
            dist = lambda e: abs(math.log2(e[0] / m)) + abs(math.log2(e[1] / n))
            best = min(dist(e) for e in entries)
            allowed = {e[2] for e in entries if abs(dist(e) - best) < 1e-9}  # ties: any of them
            assert T.trsm_lln_select_ib(dt, m, n) in allowed, (dt, m, n)


def test_python_binding_rejects_host_tensors(T):
    """Host (CPU) tensors never reach the library: their pointers would be
    taken as device addresses by the kernels.  Every binding raises before
    it calls into the library (no GPU is needed, and none is touched)."""
    import torch
    A = torch.zeros(70, 70, dtype=torch.float64).T
    B = torch.zeros(3, 70, dtype=torch.float64).T
    for call_ in (lambda: T.trsm_lln(A, B, 1.0),
                  lambda: T.trsm_lln_ex(A, B, 1.0, ib=64),
                  lambda: T.trsm_solve(A, B, 1.0, side="L", uplo="U", trans="T"),
                  lambda: T.trsm_lln_strided_batched(A.unsqueeze(0), B.unsqueeze(0), 1.0),
                  lambda: T.trsm_kernel_diag_inv(A, torch.zeros(2 * 64 * 64, dtype=torch.float64), 64),
                  lambda: T.trsm_kernel_gemm(A, B, torch.zeros(3, 70, dtype=torch.float64).T[:70])):
        with pytest.raises(ValueError, match="GPU tensor"):
            call_()


class _FakeGpuTensor:
    """Stands in for a GPU tensor in the binding's device checks (no GPU
    here): only is_cuda, get_device() and device are read."""

    def __init__(self, index):
        import torch
        self.is_cuda = True
        self._index = index
        self.device = torch.device("cuda", index)

    def get_device(self):
        return self._index


class _FakeStream:
    def __init__(self, index):
        import torch
        self.device = torch.device("cuda", index)


def test_device_checks_refuse_mixed_devices(T, monkeypatch):
    """The binding's device checks with integer device indices: operands on
    two devices, operands off the current device and a stream on another
    device are refused; matching operands give their device index; no
    operand gives None."""
    import torch
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    a0, a1 = _FakeGpuTensor(0), _FakeGpuTensor(1)
    assert T._check_device("t", a0, a0, None) == 0
    assert T._check_device("t", None, None) is None
    with pytest.raises(ValueError, match="different devices"):
        T._check_device("t", a0, a1)
    with pytest.raises(ValueError, match="current device"):
        T._check_device("t", a1, a1)
    with pytest.raises(ValueError, match="stream on"):
        T._check_device("t", a0, a0, stream=_FakeStream(1))
    assert T._check_device("t", a0, stream=_FakeStream(0)) == 0
    with pytest.raises(ValueError, match="GPU tensor"):
        T._check_device("t", a0, torch.zeros(2))


def test_noalloc_refuses_before_any_hip_call(T):
    """trsm_lln_noalloc checks its arguments like trsm_lln, and refuses a
    problem whose blocked-path workspace exceeds its fixed scratch array
    (TRSM_NOALLOC_MAX_WORKSPACE_BYTES) before any HIP call: with no GPU here,
    a HIP call would fail with HIP_ERROR instead of INVALID_VALUE."""
    al = T.alpha_buffer(1, 1.0)
    a = ctypes.addressof(al)
    f = T.lib.trsm_lln_noalloc
    assert f(1, 4, 3, a, FAKE, 3, FAKE, 4, None) == 1          # lda < m
    assert f(7, 4, 3, a, FAKE, 4, FAKE, 4, None) == 1          # dtype
    assert f(1, 0, 3, a, None, 1, None, 1, None) == 0          # m == 0
    # m = 65, n = 2^21 fp64: the panel alone is ib * n * 8 >= 1 GiB
    assert f(1, 65, 1 << 21, a, FAKE, 65, FAKE, 65, None) == 1
    # complex fp64 8192 x 2048 (ib 1024): 128 MiB of inverses + 32 MiB of panel
    alz = T.alpha_buffer(2, 1.0)
    assert f(2, 8192, 2048, ctypes.addressof(alz), FAKE, 8192, FAKE, 8192, None) == 1
