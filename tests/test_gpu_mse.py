"""TurboQuant-MSE plans and dequantization through the C ABI against the fp64 oracle.

MSE records (all b bits on the Lloyd-Max codebook, no QJL stage) against the oracle's
encode; tq_dequantize, on the library's own codes, against the oracle's reconstruction of
the same stored codes (MSE plans, inner-product plans' first stage, outlier splits), in
fp32 and bf16, with strided output rows."""
import math

import numpy as np
import pytest

from oracle import codebook, layout
from oracle import turboquant as otq
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d,bits,n,dtype", [
    (128, 3, 1001, "bfloat16"), (128, 1, 300, "float32"), (128, 4, 257, "bfloat16"),
    (128, 2, 515, "float32"), (64, 2, 200, "float32"), (32, 4, 129, "bfloat16"),
    (100, 3, 517, "float32"), (256, 3, 300, "bfloat16"), (512, 2, 70, "float32"),
    (1536, 3, 130, "float32"), (2048, 4, 40, "bfloat16"), (33, 1, 70, "bfloat16"),
    (1, 2, 65, "float32")])
def test_mse_encode_and_dequantize_match_oracle(d, bits, n, dtype):
    rng = np.random.default_rng(d * 3 + bits)
    xs = rng.standard_normal((n, d)).astype(np.float32)
    if d == 1:
        xs = np.rint(4 * xs).astype(np.float32)      # exact rotated values (see the IP test)
    xs[0] = 0.0
    x = torch.from_numpy(xs).to(DEV).to(getattr(torch, dtype))
    plan = tq.tq_plan_create_mse(d, bits, 7)
    op = otq.make_mse_plan(d, bits, 7)
    assert plan.desc["mode"] == "mse"
    sub = plan.desc["sub"][0]
    assert (sub["R"], sub["k"], sub["D"]) == (bits, 0, op.D)
    assert plan.record_bytes == layout.record_bytes_mse(op.D, bits)
    codes = tq.tq_encode(plan, x)
    torch.cuda.synchronize()
    got = layout.unpack_mse(codes.cpu().numpy(), op.D, bits)
    ref = otq.encode_mse(op, _np(x))
    parity.compare_codes_mse(op, ref, got, "mse d=%d b=%d" % (d, bits))
    # reconstruction of the stored codes, fp32 and bf16, contiguous and strided
    stored = dict(idx=got["idx"], norm=got["norm"])
    xr = otq.dequantize(op, stored)
    for odt in (torch.float32, torch.bfloat16):
        xh = tq.tq_dequantize(plan, codes, n, dtype=odt)
        wide = torch.full((n, d + 5), 7.0, dtype=odt, device=DEV)
        tq.tq_dequantize(plan, codes, n, x=wide[:, :d])
        torch.cuda.synchronize()
        parity.check_dequantized(_np(xh), xr, got["norm"], odt == torch.bfloat16,
                                 "dequant d=%d b=%d %s" % (d, bits, odt))
        assert torch.equal(wide[:, :d], xh) and bool(torch.all(wide[:, d:] == 7.0))
    assert np.all(_np(xh)[0] == 0.0)


def test_mse_distortion_on_gpu_matches_analytic():
    """3-bit MSE at d = D = 128: mean ||u - uhat||^2 over uniform directions equals D times
    the codebook's per-coordinate MSE within 3 standard errors."""
    d, b, n = 128, 3, 20000
    rng = np.random.default_rng(1)
    xs = rng.standard_normal((n, d))
    xs /= np.linalg.norm(xs, axis=1, keepdims=True)
    x = torch.from_numpy(xs.astype(np.float32)).to(DEV)
    plan = tq.tq_plan_create_mse(d, b, 3)
    xh = _np(tq.tq_dequantize(plan, tq.tq_encode(plan, x), n))
    err = np.sum((_np(x) - xh) ** 2, axis=1)
    op = otq.make_mse_plan(d, b, 3)
    analytic = d * codebook.codebook_mse(d, op.levels, op.thresholds)
    assert abs(err.mean() - analytic) < 3 * err.std() / math.sqrt(n)


@pytest.mark.parametrize("d,bits,mask", [(128, 4, False), (1536, 3, False), (128, 3, True)])
def test_dequantize_inner_product_plans(d, bits, mask):
    """An inner-product plan reconstructs its (b-1)-bit first stage; an outlier split writes
    each sub-plan's channels."""
    rng = np.random.default_rng(d + bits)
    n = 300
    xs = rng.standard_normal((n, d)).astype(np.float32)
    if mask:
        m = np.zeros(d, dtype=np.uint8)
        m[rng.choice(d, 32, replace=False)] = 1
        plan = tq.tq_plan_create(d, bits, 5, m, bits + 2)
        sp = otq.make_split_plan(d, bits, 5, m, bits + 2)
    else:
        plan = tq.tq_plan_create(d, bits, 5)
        sp = otq.make_split_plan(d, bits, 5)
    codes = tq.tq_encode(plan, torch.from_numpy(xs).to(DEV))
    xh = tq.tq_dequantize(plan, codes, n)
    torch.cuda.synchronize()
    got = layout.unpack_split(sp, codes.cpu().numpy())
    xr = otq.dequantize_split(sp, got)
    norms = np.sqrt(sum(g["norm"] ** 2 for g in got))
    parity.check_dequantized(_np(xh), xr, norms, False, "ip dequant d=%d" % d)


def test_mse_plan_rejects_bad_arguments():
    """Bit widths outside 1..4 and lengths above 2048 are refused (scoring MSE records is
    tested in tests/test_gpu_mse_score.py)."""
    for bits in (0, 5):
        with pytest.raises(tq.TqError):
            tq.tq_plan_create_mse(128, bits, 0)
    with pytest.raises(tq.TqError):
        tq.tq_plan_create_mse(4096, 3, 0)


def test_dequantize_every_mfma_shape():
    """Every (D <= 128, b) combination of the matrix-core reconstruction, fp32 and bf16 out
    (each is its own compiled kernel)."""
    for d in (32, 64, 128):
        for bits in (1, 2, 3, 4):
            rng = np.random.default_rng(d + 10 * bits)
            xs = rng.standard_normal((97, d)).astype(np.float32)
            plan = tq.tq_plan_create_mse(d, bits, 13)
            op = otq.make_mse_plan(d, bits, 13)
            codes = tq.tq_encode(plan, torch.from_numpy(xs).to(DEV))
            got = layout.unpack_mse(codes.cpu().numpy(), op.D, bits)
            xr = otq.dequantize(op, dict(idx=got["idx"], norm=got["norm"]))
            for odt in (torch.float32, torch.bfloat16):
                xh = tq.tq_dequantize(plan, codes, 97, dtype=odt)
                parity.check_dequantized(_np(xh), xr, got["norm"], odt == torch.bfloat16,
                                         "dequant D=%d b=%d %s" % (d, bits, odt))
