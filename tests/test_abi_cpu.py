"""Host-side tests of the C ABI: the library loads, exports every function
``include/muon.h`` declares, sizes workspaces, and rejects bad arguments
before anything is enqueued (these paths make no HIP call, so they run on a
machine without a GPU)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from matrix_orthogonalizing_optimizer_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mo_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_abi():
    names = _declared_functions()
    for required in ["mo_muon_step", "mo_adamw_step", "mo_newton_schulz",
                     "mo_muon_workspace_size", "mo_last_error", "mo_muon_plan_create",
                     "mo_muon_plan_step", "mo_muon_plan_destroy"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding's signature table covers them all
    assert set(_declared_functions()) == set(L._SIGS)


def test_abi_version():
    src = open(HEADER).read()
    v = int(re.search(r"#define MO_ABI_VERSION (\d+)", src).group(1))
    assert L.lib().mo_abi_version() == v


def _tensors(shapes, base=0x10000000, grad_size=2, mom_size=2, state1=False):
    arr = (L.MoTensor * max(1, len(shapes)))()
    off = base
    for i, (r, c) in enumerate(shapes):
        n = r * c
        arr[i].param = off
        off += (n * 4 + 255) // 256 * 256
        arr[i].grad = off
        off += (n * grad_size + 255) // 256 * 256
        arr[i].state0 = off
        off += (n * mom_size + 255) // 256 * 256
        if state1:
            arr[i].state1 = off
            off += (n * 4 + 255) // 256 * 256
        arr[i].rows, arr[i].cols = r, c
    return arr


def _ws(shapes, ns=L.MO_BF16):
    full, mn = ctypes.c_size_t(), ctypes.c_size_t()
    rc = L.lib().mo_muon_workspace_size(_tensors(shapes), len(shapes), ns,
                                        ctypes.byref(full), ctypes.byref(mn))
    return rc, full.value, mn.value


def test_workspace_size_query():
    rc, full, mn = _ws([(1536, 1536)] * 4 + [(1536, 6144)] * 2)
    assert rc == L.MO_OK
    assert full >= mn > 0
    # one 1536x6144 bf16 matrix needs its two iterates and the m x m S and P
    def need(m, n, esz):
        return (2 * m * n + 2 * m * m) * esz
    assert mn >= need(1536, 6144, 2)
    # the full size holds every matrix of every shape group at once
    assert full >= 4 * need(1536, 1536, 2) + 2 * need(1536, 6144, 2)
    rc, full32, mn32 = _ws([(128, 512)], L.MO_F32)
    assert rc == L.MO_OK and mn32 >= need(128, 512, 4)
    # orientation does not change the requirement
    assert _ws([(6144, 1536)])[1:] == _ws([(1536, 6144)])[1:]


def test_workspace_grows_with_count():
    _, f1, m1 = _ws([(512, 2048)])
    _, f8, m8 = _ws([(512, 2048)] * 8)
    assert m8 == m1 and f8 > f1


def _step(arr, n, gdt=L.MO_BF16, mdt=L.MO_BF16, ndt=L.MO_BF16, lr=1e-3, wd=0.1, mu=0.95,
          ns_steps=5, eps=1e-7, ws=0x70000000, ws_bytes=1 << 40, rms=None):
    return L.lib().mo_muon_step(arr, n, gdt, mdt, ndt, lr, wd, mu, 1, ns_steps, None, 0.2, eps,
                                rms, ws, ws_bytes, None)


@pytest.mark.parametrize("case,code", [
    ("bad_grad_dtype", L.MO_EINVAL), ("bad_ns_dtype", L.MO_EINVAL),
    ("negative_count", L.MO_EINVAL), ("null_tensors", L.MO_EINVAL),
    ("zero_rows", L.MO_EINVAL), ("null_param", L.MO_EINVAL),
    ("misaligned_grad", L.MO_EINVAL), ("state1_set", L.MO_EINVAL),
    ("overlap", L.MO_EINVAL), ("ns_steps_17", L.MO_EINVAL),
    ("ns_steps_neg", L.MO_EINVAL), ("nan_lr", L.MO_EINVAL), ("neg_eps", L.MO_EINVAL),
    ("null_workspace", L.MO_EWORKSPACE), ("small_workspace", L.MO_EWORKSPACE),
    ("misaligned_workspace", L.MO_EWORKSPACE), ("misaligned_rms", L.MO_EINVAL),
])
def test_muon_step_rejects(case, code):
    shapes = [(64, 128), (128, 64)]
    arr = _tensors(shapes)
    kw = {}
    n = len(shapes)
    if case == "bad_grad_dtype":
        kw["gdt"] = 7
    elif case == "bad_ns_dtype":
        kw["ndt"] = -1
    elif case == "negative_count":
        n = -1
    elif case == "null_tensors":
        arr = None
    elif case == "zero_rows":
        arr[1].rows = 0
    elif case == "null_param":
        arr[0].param = None
    elif case == "misaligned_grad":
        arr[1].grad = arr[1].grad + 4
    elif case == "state1_set":
        arr[0].state1 = 0x50000000
    elif case == "overlap":
        arr[1].state0 = arr[0].param + 64
    elif case == "ns_steps_17":
        kw["ns_steps"] = 17
    elif case == "ns_steps_neg":
        kw["ns_steps"] = -1
    elif case == "nan_lr":
        kw["lr"] = float("nan")
    elif case == "neg_eps":
        kw["eps"] = -1.0
    elif case == "null_workspace":
        kw["ws"] = None
    elif case == "small_workspace":
        kw["ws_bytes"] = 1024
    elif case == "misaligned_workspace":
        kw["ws"] = 0x70000010
    elif case == "misaligned_rms":
        kw["rms"] = 0x60000002
    rc = _step(arr, n, **kw)
    assert rc == code, (rc, L.last_error())
    assert L.last_error()


def test_empty_step_is_ok_without_workspace():
    assert _step(None, 0, ws=None, ws_bytes=0) == L.MO_OK


@pytest.mark.parametrize("case", ["null_v", "zero_step", "beta1_one", "misaligned_m",
                                  "bad_dtype", "overlap", "inf_wd"])
def test_adamw_rejects(case):
    arr = _tensors([(1, 1000), (1, 77)], grad_size=4, mom_size=4, state1=True)
    gdt, step, b1, wd = L.MO_F32, 1, 0.9, 0.1
    if case == "null_v":
        arr[1].state1 = None
    elif case == "zero_step":
        step = 0
    elif case == "beta1_one":
        b1 = 1.0
    elif case == "misaligned_m":
        arr[0].state0 = arr[0].state0 + 8
    elif case == "bad_dtype":
        gdt = 3
    elif case == "overlap":
        arr[1].param = arr[0].state1
    elif case == "inf_wd":
        wd = float("inf")
    rc = L.lib().mo_adamw_step(arr, 2, gdt, 1e-3, wd, b1, 0.999, 1e-8, step, None)
    assert rc == L.MO_EINVAL, L.last_error()


def test_newton_schulz_rejects_overlap_and_bad_args():
    lib = L.lib()
    rc = lib.mo_newton_schulz(0x10000000, 0x10000100, 2, 64, 64, L.MO_BF16, 5, None, 1e-7,
                              0x70000000, 1 << 40, None)
    assert rc == L.MO_EINVAL
    rc = lib.mo_newton_schulz(0x10000000, 0x20000000, 1, 64, 64, L.MO_BF16, 99, None, 1e-7,
                              0x70000000, 1 << 40, None)
    assert rc == L.MO_EINVAL
    rc = lib.mo_newton_schulz(0x10000000, 0x20000000, 1, 64, 64, L.MO_BF16, 5, None, 1e-7,
                              0x70000000, 100, None)
    assert rc == L.MO_EWORKSPACE
    out = ctypes.c_size_t()
    assert lib.mo_newton_schulz_workspace_size(3, 100, 300, L.MO_F32, ctypes.byref(out)) == 0
    # two iterates and S, P for each of the three matrices (at least the true sizes)
    assert out.value > 3 * (2 * 100 * 300 + 2 * 100 * 100) * 4


def test_plan_create_rejects_before_allocating():
    h = ctypes.c_void_p()
    arr = _tensors([(64, 64)])
    arr[0].grad = arr[0].param   # alias
    rc = L.lib().mo_muon_plan_create(arr, 1, L.MO_BF16, L.MO_BF16, L.MO_BF16, ctypes.byref(h))
    assert rc == L.MO_EINVAL and not h.value


def test_profile_counters_host_side():
    lib = L.lib()
    assert lib.mo_profile_enable(0) == 0
    n, ms, w = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
    assert lib.mo_profile_read(L.MO_K_UPDATE, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(w)) == 0
    assert lib.mo_profile_read(42, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(w)) == L.MO_EINVAL
    assert lib.mo_profile_reset() == 0


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "matrix_orthogonalizing_optimizer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in re.sub(r"#.*|//.*", "", txt).lower().replace(
                    "oracle_", ""), f


def _mats(shapes, base=0x10000000):
    arr = (L.MoMatrix * max(len(shapes), 1))()
    off = base
    for i, (r, c) in enumerate(shapes):
        arr[i].data, arr[i].rows, arr[i].cols = off, r, c
        off += (r * c * 4 + 255) // 256 * 256
    return arr


def _svd_ws(shapes):
    full, mn = ctypes.c_size_t(), ctypes.c_size_t()
    rc = L.lib().mo_svd_entropy_workspace_size(_mats(shapes), len(shapes), ctypes.byref(full),
                                               ctypes.byref(mn))
    return rc, full.value, mn.value


def test_svd_entropy_workspace_size():
    rc, full, mn = _svd_ws([(1536, 1536)] * 4 + [(6144, 1536)] * 2 + [(64, 2048)])
    assert rc == L.MO_OK
    # one m x m fp64 working matrix per matrix plus vectors; the m = 1536
    # group (6 matrices, both orientations) is the largest chunk
    assert mn >= 1536 * 1536 * 8 and full >= 6 * 1536 * 1536 * 8
    # plus v (2), the panel's v and w (2 x 16), d, e, eigenvalues per row
    assert full < 6 * 1536 * (1536 + 1536 // 64 + 40) * 8 + 4096
    assert _svd_ws([(300, 40)])[1:] == _svd_ws([(40, 300)])[1:]
    assert _svd_ws([(8193, 8193)])[0] == L.MO_EINVAL
    assert _svd_ws([(8192, 1 << 18)])[0] == L.MO_OK
    assert _svd_ws([(8192, (1 << 18) + 1)])[0] == L.MO_EINVAL
    assert _svd_ws([(1, (1 << 31) - 1)])[0] == L.MO_OK
    assert _svd_ws([((1 << 31), 1)])[0] == L.MO_EINVAL        # a side must fit in 32 bits


@pytest.mark.parametrize("case,code", [
    ("bad_dtype", L.MO_EINVAL), ("negative_count", L.MO_EINVAL), ("null_mats", L.MO_EINVAL),
    ("zero_cols", L.MO_EINVAL), ("null_data", L.MO_EINVAL), ("misaligned_data", L.MO_EINVAL),
    ("too_wide", L.MO_EINVAL), ("null_entropy", L.MO_EINVAL), ("misaligned_sigma", L.MO_EINVAL),
    ("sigma_overlaps_input", L.MO_EINVAL), ("entropy_overlaps_sigma", L.MO_EINVAL),
    ("ws_overlaps_input", L.MO_EINVAL), ("null_workspace", L.MO_EWORKSPACE),
    ("small_workspace", L.MO_EWORKSPACE),
])
def test_svd_entropy_rejects(case, code):
    shapes = [(64, 128), (200, 96)]
    arr = _mats(shapes)
    n, dt = len(shapes), L.MO_F32
    ent, sig, ws, ws_bytes = 0x50000000, 0x51000000, 0x70000000, 1 << 40
    if case == "bad_dtype":
        dt = 3
    elif case == "negative_count":
        n = -1
    elif case == "null_mats":
        arr = None
    elif case == "zero_cols":
        arr[1].cols = 0
    elif case == "null_data":
        arr[0].data = None
    elif case == "misaligned_data":
        arr[1].data = arr[1].data + 8
    elif case == "too_wide":
        arr[0].rows, arr[0].cols = 9000, 9000
    elif case == "null_entropy":
        ent = None
    elif case == "misaligned_sigma":
        sig = 0x51000004
    elif case == "sigma_overlaps_input":
        sig = arr[1].data + 64
    elif case == "entropy_overlaps_sigma":
        ent = sig + 8
    elif case == "ws_overlaps_input":
        ws = 0x10000000 - 256
    elif case == "null_workspace":
        ws = None
    elif case == "small_workspace":
        ws_bytes = 4096
    rc = L.lib().mo_svd_entropy(arr, n, dt, ent, sig, ws, ws_bytes, None)
    assert rc == code, (rc, L.last_error())
    assert L.last_error()


def test_svd_entropy_empty_call_is_ok():
    assert L.lib().mo_svd_entropy(None, 0, L.MO_F32, None, None, None, 0, None) == L.MO_OK
