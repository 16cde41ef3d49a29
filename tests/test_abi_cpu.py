"""The C-ABI library without a GPU: it loads, exports every entry point that
include/mfpcg.h declares, and rejects invalid arguments before any GPU work."""
import ctypes
import os
import re

import numpy as np
import pytest

from matrix_free_pcg_amd import _abi
from matrix_free_pcg_amd import build as hipbuild

HEADER = os.path.join(hipbuild.INCLUDE, "mfpcg.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hipbuild.LIB) or hipbuild.is_stale():
        hipbuild.build()
    return _abi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pcg_[A-Za-z0-9_]+)\s*\(", text)))


def test_header_declares_the_contract():
    names = declared_functions()
    for required in ("pcg_create", "pcg_destroy", "pcg_apply_A", "pcg_precond", "pcg_solve",
                     "pcg_last_error", "pcg_solve_workspace_bytes"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(_abi.EXPORTED) == names


def test_version_and_error_strings(lib):
    assert "gfx950" in _abi.pcg_version()
    assert isinstance(_abi.pcg_last_error(None), str)


# a stand-in for a device table buffer: 256-byte aligned and large enough;
# never dereferenced (every case below fails before any HIP call)
FAKE_TABLES = 1 << 40


def _create(lib, nx, ny, nz, delta, az, kind=0, hconst=1.0, field=None, tables=FAKE_TABLES, tbytes=1 << 30):
    g = _abi.pcg_grid(nx, ny, nz)
    c = _abi.pcg_coeffs()
    c.delta = delta
    az = np.ascontiguousarray(az, dtype=np.float64)
    c.alpha_z_face = az.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    c.alpha_h_kind = kind
    c.alpha_h_const = hconst
    if field is not None:
        field = np.ascontiguousarray(field, dtype=np.float64)
        c.alpha_h_field = field.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    out = ctypes.c_void_p()
    rc = lib.pcg_create(ctypes.byref(g), ctypes.byref(c), None, tables, tbytes, ctypes.byref(out))
    return rc, out.value, (az, field)


@pytest.mark.parametrize("case,expect", [
    ("delta_zero", _abi.PCG_ERR_INVALID),
    ("delta_nan", _abi.PCG_ERR_INVALID),
    ("face_negative", _abi.PCG_ERR_INVALID),
    ("boundary_face", _abi.PCG_ERR_INVALID),
    ("nz_zero", _abi.PCG_ERR_INVALID),
    ("nx_negative", _abi.PCG_ERR_INVALID),
    ("nz_too_big", _abi.PCG_ERR_UNSUPPORTED),
    ("alpha_h_negative", _abi.PCG_ERR_INVALID),
    ("field_negative", _abi.PCG_ERR_INVALID),
    ("field_null", _abi.PCG_ERR_INVALID),
    ("bad_kind", _abi.PCG_ERR_INVALID),
    ("tables_null", _abi.PCG_ERR_INVALID),
    ("tables_misaligned", _abi.PCG_ERR_INVALID),
    ("tables_short", _abi.PCG_ERR_INVALID),
])
def test_create_rejects_invalid_arguments(lib, case, expect):
    nz = 8
    az = np.zeros(nz + 1)
    az[1:nz] = 10.0
    args = dict(nx=4, ny=4, nz=nz, delta=1e-2, az=az)
    if case == "delta_zero":
        args["delta"] = 0.0
    elif case == "delta_nan":
        args["delta"] = float("nan")
    elif case == "face_negative":
        az[3] = -1.0
    elif case == "boundary_face":
        az[0] = 1.0
    elif case == "nz_zero":
        args["nz"] = 0
        args["az"] = np.zeros(1)
    elif case == "nx_negative":
        args["nx"] = -3
    elif case == "nz_too_big":
        args["nz"] = 513
        args["az"] = np.zeros(514)
    elif case == "alpha_h_negative":
        args["hconst"] = -0.5
    elif case == "field_negative":
        f = np.ones((4, 4))
        f[2, 1] = -1.0
        args.update(kind=1, field=f)
    elif case == "field_null":
        args.update(kind=1)
    elif case == "bad_kind":
        args.update(kind=7)
    elif case == "tables_null":
        args.update(tables=None)
    elif case == "tables_misaligned":
        args.update(tables=FAKE_TABLES + 8)
    elif case == "tables_short":
        g = _abi.pcg_grid(4, 4, nz)
        args.update(tbytes=lib.pcg_handle_bytes(ctypes.byref(g)) - 1)
    rc, h, _keep = _create(lib, **args)
    assert rc == expect
    assert h is None
    assert len(_abi.pcg_last_error(None)) > 0
    if case.startswith("tables"):
        assert "tables_dev" in _abi.pcg_last_error(None)


def test_handle_bytes_covers_the_tables(lib):
    """pcg_handle_bytes: the handle's device tables (faces, a and d per level,
    |T| and two edges per column, binary64 and binary32 multipliers at the
    segment boundaries, each part rounded up to 256 bytes), 0 for an invalid
    grid; no device memory is allocated by the library."""
    def a256(b):
        return (b + 255) // 256 * 256
    for nx, ny, nz in [(32, 32, 16), (1024, 1024, 128), (5, 3, 7), (64, 8, 300)]:
        g = _abi.pcg_grid(nx, ny, nz)
        L = 8 if nz <= 128 else (16 if nz <= 256 else 32)
        P = -(-nz // L)
        ncol = nx * ny
        nb = ncol * max(P - 1, 1)
        want = a256(8 * (nz + 1)) + a256(8 * (2 * nz + 3 * ncol)) + a256(8 * nb) + a256(4 * nb)
        assert lib.pcg_handle_bytes(ctypes.byref(g)) == want, (nx, ny, nz)
    for bad in [(0, 4, 4), (4, -1, 4), (4, 4, 0), (4, 4, 513)]:
        g = _abi.pcg_grid(*bad)
        assert lib.pcg_handle_bytes(ctypes.byref(g)) == 0
    assert lib.pcg_handle_bytes(None) == 0



def test_tuning_variables_agree():
    """The tuning variables are the same set in the header (a PCG_TUNE_*
    bit and a line in its list each), in the binding's name table and in
    the environment variables the library reads, each with the bit it
    reports."""
    header = open(HEADER).read()
    bits = {int(v, 16): "MFPCG_" + n for n, v in re.findall(r"#define PCG_TUNE_(\w+) (0x[0-9A-Fa-f]+)", header)}
    assert bits and bits == _abi.PCG_TUNE_NAMES
    src = re.sub(r"//[^\n]*", "", open(os.path.join(hipbuild.CSRC, "mfpcg.hip")).read())
    read = dict(re.findall(r'env_int\("(MFPCG_\w+)",[^;]*?PCG_TUNE_(\w+)\)', src, flags=re.S))
    for bit, name in bits.items():
        assert name in header.split("#define PCG_TUNE_")[0], name   # listed in the header's comment
        assert read.get(name) == name[len("MFPCG_"):], (name, read.get(name))
    assert set(read) == set(bits.values())

def test_no_device_allocation_in_the_library():
    """The library's source makes no device allocation: no hipMalloc /
    hipFree / hipMallocAsync / hipExtMalloc call in the host code (the pinned
    status word is hipHostMalloc'ed host memory)."""
    import re as _re
    src = open(os.path.join(hipbuild.CSRC, "mfpcg.hip")).read()
    src = _re.sub(r"//[^\n]*", "", src)
    for name in ("hipMalloc(", "hipMallocManaged", "hipMallocAsync", "hipExtMallocWithFlags", "hipFree("):
        assert name not in src, name


def test_static_solve_contract_without_gpu(lib):
    assert lib.pcg_solve_static_max_bytes() == 64 << 20
    assert lib.pcg_solve_static(None, None, None, 1e-8, 10, None, None, None, None) == _abi.PCG_ERR_INVALID
    assert lib.pcg_tuning_overrides(None) == 0
    assert lib.pcg_tridiag_bytes(None) == 0
    p = _abi.pcg_mg_params(1, 0.8, 0, 2)
    assert lib.pcg_mg_setup_bytes(None, ctypes.byref(p)) == 0


def test_null_handle_calls_are_invalid(lib):
    assert lib.pcg_apply_A(None, None, None) == _abi.PCG_ERR_INVALID
    assert lib.pcg_precond(None, None, None) == _abi.PCG_ERR_INVALID
    assert lib.pcg_destroy(None) == _abi.PCG_OK
    assert lib.pcg_solve_workspace_bytes(None, 10) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(hipbuild, "LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _abi.load()


@pytest.mark.parametrize("case", ["a_zero", "a_nan", "d_negative", "beta_boundary", "beta_negative",
                                  "area_zero", "alpha_x_negative", "alpha_y_inf", "null_area"])
def test_create_general_rejects_invalid_arguments(lib, case):
    nx, ny, nz = 4, 3, 6
    arrs = dict(a=np.full(nz, 1e-2), d=np.ones(nz), beta_face=np.r_[0.0, np.full(nz - 1, 5.0), 0.0],
                area=np.ones(nx * ny), alpha_x=np.ones(nx * ny), alpha_y=np.ones(nx * ny))
    if case == "a_zero":
        arrs["a"][2] = 0.0
    elif case == "a_nan":
        arrs["a"][0] = float("nan")
    elif case == "d_negative":
        arrs["d"][1] = -1.0
    elif case == "beta_boundary":
        arrs["beta_face"][nz] = 1.0
    elif case == "beta_negative":
        arrs["beta_face"][3] = -2.0
    elif case == "area_zero":
        arrs["area"][5] = 0.0
    elif case == "alpha_x_negative":
        arrs["alpha_x"][0] = -0.1
    elif case == "alpha_y_inf":
        arrs["alpha_y"][7] = float("inf")
    c = _abi.pcg_coeffs_general()
    for name, v in arrs.items():
        if case == "null_area" and name == "area":
            continue
        setattr(c, name, v.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    g = _abi.pcg_grid(nx, ny, nz)
    out = ctypes.c_void_p()
    rc = lib.pcg_create_general(ctypes.byref(g), ctypes.byref(c), None, FAKE_TABLES, 1 << 30, ctypes.byref(out))
    assert rc == _abi.PCG_ERR_INVALID
    assert out.value is None
    assert "pcg_create_general" in _abi.pcg_last_error(None)


def test_mg_entry_points_reject_null_handle(lib):
    p = _abi.pcg_mg_params(1, 0.8, 0, 2)
    assert lib.pcg_mg_setup(None, ctypes.byref(p), None, 0) == _abi.PCG_ERR_INVALID
    n = ctypes.c_int32(0)
    assert lib.pcg_mg_num_levels(None, ctypes.byref(n)) == _abi.PCG_ERR_INVALID
    assert lib.pcg_mg_level(None, 0, None, None, None, None, None) == _abi.PCG_ERR_INVALID
    assert lib.pcg_mg_workspace_bytes(None, 10) == 0
    assert lib.pcg_mg_vcycle(None, None, None, None, 0) == _abi.PCG_ERR_INVALID
    assert lib.pcg_solve_mg(None, None, None, 1e-8, 10, None, 0, None, None, None, None) == _abi.PCG_ERR_INVALID


def test_stream_probe_rejects_bad_arguments():
    """The bandwidth probe that bench.py --stream-probe loads (a measurement
    tool beside the solver) rejects invalid stream counts and sizes on the host
    (return -1, nothing launched)."""
    if not os.path.exists(hipbuild.PROBE_LIB):
        hipbuild.build()
    probe = ctypes.CDLL(hipbuild.PROBE_LIB)
    for f in (probe.mfprobe_stream, probe.mfprobe_stream_f32):   # float64 and float32 elements
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_int64, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                      ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
        ins = (ctypes.c_void_p * 5)(*([ctypes.c_void_p(4096)] * 5))
        outs = (ctypes.c_void_p * 3)(*([ctypes.c_void_p(8192)] * 3))
        ms = ctypes.c_double(0.0)
        for r, w, e, b, n, reps in [(0, 1, 4, 256, 1024, 1), (8, 1, 4, 256, 1024, 1), (1, 0, 4, 256, 1024, 1),
                                    (1, 4, 4, 256, 1024, 1), (1, 1, 3, 256, 1024, 1), (1, 1, 4, 100, 1024, 1),
                                    (1, 1, 4, 2048, 8192, 1), (1, 1, 4, 256, 1000, 1), (1, 1, 4, 256, 0, 1),
                                    (1, 1, 4, 256, 1024, 0)]:
            assert f(r, w, 1, e, b, n, ins, outs, reps, None, ctypes.byref(ms)) == -1, (r, w, e, b, n, reps)
        nulls = (ctypes.c_void_p * 5)()
        assert f(2, 1, 1, 4, 256, 1024, nulls, outs, 1, None, ctypes.byref(ms)) == -1
