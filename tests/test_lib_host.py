"""CPU tests of the C-ABI library: symbols, host-side plan tables against the
oracle, and argument validation (no compute call needs a GPU here)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import rotation_online_vector_amd as tq
from oracle import codebook, philox

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_header_function():
    lib = tq.load_library()
    names = _header_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(tq.EXPORTED) == names


@pytest.mark.parametrize("D,R", [(128, 3), (128, 2), (128, 1), (32, 4), (32, 3), (2048, 3), (64, 2),
                                 (3, 2), (256, 4)])
def test_library_codebook_matches_oracle(D, R):
    lv, th = tq.tq_codebook(D, R)
    olv, oth = codebook.solve_codebook(D, R)
    s = 1 / math.sqrt(D)
    # the oracle stops its plain Lloyd iteration once a step moves < 1e-13 s; at R = 4 the
    # iteration contracts by ~0.96 per step, leaving ~3e-12 s to the fixed point
    assert np.max(np.abs(lv - olv)) < 1e-11 * s
    assert np.max(np.abs(th - oth)) < 1e-11 * s
    # exact mirror symmetry with the middle threshold at 0, also after rounding to fp32 (the
    # encode kernels quantize |z| against the positive half and take the sign separately)
    assert np.array_equal(lv, -lv[::-1])
    assert np.array_equal(th, -th[::-1]) and th[(1 << R) // 2 - 1] == 0.0
    lf, tf = lv.astype(np.float32), th.astype(np.float32)
    assert np.array_equal(lf, -lf[::-1]) and np.array_equal(tf, -tf[::-1])


@pytest.mark.parametrize("seed,subset,D", [(0, 0, 128), (0, 1, 32), (123456789123, 0, 2048),
                                           (2 ** 64 - 1, 1, 64)])
def test_library_rotation_signs_match_oracle(seed, subset, D):
    assert np.array_equal(tq.tq_rotation_signs(seed, subset, D),
                          philox.rotation_signs(seed, subset, D).astype(np.int8))


@pytest.mark.parametrize("seed,subset,k,D", [(0, 0, 128, 128), (0, 1, 32, 32), (7, 0, 2048, 2048),
                                             (5, 1, 3, 5)])
def test_library_qjl_matrix_matches_oracle_bits(seed, subset, k, D):
    lib_bits = tq.tq_qjl_matrix(seed, subset, k, D)
    ora_bits = philox.bf16_bits(philox.qjl_matrix(seed, subset, k, D))
    assert np.array_equal(lib_bits, ora_bits)


def test_status_strings():
    lib = tq.load_library()
    for st in (0, -1, -2, -3, -4):
        assert lib.tq_status_string(st)
    assert lib.tq_status_string(0) == b"ok"


def _create(d, bits, mask=None, obits=0):
    lib = tq.load_library()
    h = ctypes.c_void_p(123)
    buf = None if mask is None else np.asarray(mask, dtype=np.uint8)
    st = lib.tq_plan_create(d, bits, 0, None if buf is None else buf.ctypes.data_as(ctypes.c_void_p),
                            obits, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("args", [(0, 3), (2049, 3), (128, 1), (128, 6)])
def test_plan_create_rejects_bad_sizes(args):
    st, h = _create(*args)
    assert st == tq.TQ_EINVAL and h.value is None


def test_plan_create_rejects_bad_masks():
    assert _create(8, 3, [0] * 8, 3)[0] == tq.TQ_EINVAL       # no outlier channel
    assert _create(8, 3, [1] * 8, 3)[0] == tq.TQ_EINVAL       # no regular channel
    assert _create(8, 3, [1] + [0] * 7, 1)[0] == tq.TQ_EINVAL  # outlier bits out of range
    assert _create(8, 3, [1] + [0] * 7, 6)[0] == tq.TQ_EINVAL
    lib = tq.load_library()
    assert lib.tq_plan_create(8, 3, 0, None, 0, None) == tq.TQ_EINVAL


def test_calls_validate_before_touching_the_device():
    lib = tq.load_library()
    assert lib.tq_encode(None, None, 0, 1, 128, None, None) == tq.TQ_EINVAL
    assert lib.tq_score(None, None, 0, 1, 1, 128, None, 1, None, None) == tq.TQ_EINVAL
    assert lib.tq_qjl(None, 0, None, 1, None, None) == tq.TQ_EINVAL
    assert lib.tq_plan_info(None, None) == tq.TQ_EINVAL
    lib.tq_plan_destroy(None)
    p = ctypes.c_void_p(16)
    assert lib.tq_topk(p, 1, 10, 0, p, p, None) == tq.TQ_EINVAL     # k < 1
    assert lib.tq_topk(p, 1, 10, 11, p, p, None) == tq.TQ_EINVAL    # k > n
    assert lib.tq_topk(p, 1, 100, 65, p, p, None) == tq.TQ_EINVAL   # k > 64
    assert lib.tq_topk(p, 0, 100, 5, None, None, None) == tq.TQ_OK  # empty
    assert lib.tq_codebook(2, 2, p, p) == tq.TQ_EINVAL
    assert lib.tq_rotation_signs(0, 0, 48, p) == tq.TQ_EINVAL       # not a power of two
    assert lib.tq_rotation_signs(0, 2, 64, p) == tq.TQ_EINVAL       # bad subset


def test_plan_create_without_device_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, h = _create(128, 3)
    assert st == tq.TQ_EDEVICE and h.value is None


def test_c_abi_from_plain_c(tmp_path):
    """The header compiles as C and the library links and answers from a plain C program
    (gcc, no HIP headers): host building blocks, status strings, argument validation."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib_dir = os.path.dirname(tq.LIB_PATH)
    exe = str(tmp_path / "c_abi_host")
    src = os.path.join(ROOT, "tests", "c", "c_abi_host.c")
    subprocess.run([gcc, "-std=c99", "-O1", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    src, "-o", exe, "-L", lib_dir, "-ltq", "-lm", "-Wl,-rpath," + lib_dir],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip().endswith("all passed")


def test_bindings_refuse_host_tensors():
    """Host tensors never reach the library: their pointers would fault the device."""
    import torch
    import rotation_online_vector_amd as tq
    q = torch.zeros((2, 16))
    x = torch.zeros((5, 16))
    cand = torch.zeros((2, 4), dtype=torch.int64)
    with pytest.raises(ValueError, match="GPU"):
        tq.tq_rerank(q, x, cand, 2)
    with pytest.raises(ValueError, match="GPU"):
        tq.tq_calibrate_outliers(x, 2)
    with pytest.raises(ValueError, match="GPU"):
        tq.tq_topk(torch.zeros((2, 8)), 2)


def test_bindings_check_caller_outputs():
    """A caller-provided output of the wrong dtype or size is refused before the library runs
    (checked on the host; the device check comes first, so CPU tensors exercise only that)."""
    import torch
    import rotation_online_vector_amd as tq
    t = torch.zeros(3, dtype=torch.float32)
    with pytest.raises(ValueError):
        tq._out(t, torch.float64, 3, "var")
    with pytest.raises(ValueError):
        tq._out(t, torch.float32, 4, "vals")
    tq._out(t, torch.float32, 3, "vals")


def test_bindings_check_code_inputs_and_group_sizes():
    """Record buffers are read as contiguous bytes: a non-uint8, non-contiguous or short
    buffer is refused; empty groups give nq_per_group 0 (the C ABI's no-op) instead of a
    division by zero, and mismatched group sizes are refused."""
    import torch
    import rotation_online_vector_amd as tq
    tq._codes(torch.zeros(56, dtype=torch.uint8), 56)
    with pytest.raises(ValueError):
        tq._codes(torch.zeros(56, dtype=torch.uint8), 57)
    with pytest.raises(ValueError):
        tq._codes(torch.zeros(14, dtype=torch.int32), 56)
    with pytest.raises(ValueError):
        tq._codes(torch.zeros((2, 56), dtype=torch.uint8).t(), 56)
    assert tq._groups(0, None, 0) == 0
    assert tq._groups(12, None, 3) == 4
    assert tq._groups(12, 6, 2) == 6
    with pytest.raises(ValueError):
        tq._groups(12, 5, 2)
    with pytest.raises(ValueError):
        tq._groups(4, None, -1)
