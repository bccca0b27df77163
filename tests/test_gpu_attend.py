"""Decode attention over quantized values (tq_attend) through the C ABI against the fp64
oracle, on the library's own value codes and the same logits: single and ragged chunks of
1024 tokens, several query tiles, every thread layout (D below, at and above the block
size), inner-product value plans, logits produced by tq_score, fp32 and bf16 output."""
import numpy as np
import pytest

from oracle import layout
from oracle import turboquant as otq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(out, ref, vmax, bf16, what):
    tol = 2e-5 * vmax + (2.0 ** -8 * np.abs(ref) if bf16 else 0.0)
    err = np.abs(out - ref)
    assert np.all(err <= tol), "%s: max err/tol %g" % (what, float(np.max(err / tol)))


@pytest.mark.parametrize("d,bits,n,nqg,groups,mode,dtype", [
    (128, 3, 5000, 4, 2, "mse", "float32"), (128, 2, 1024, 8, 1, "mse", "bfloat16"),
    (64, 4, 3000, 12, 1, "mse", "float32"), (256, 3, 2500, 4, 1, "mse", "float32"),
    (2048, 3, 700, 4, 1, "mse", "bfloat16"), (100, 4, 1500, 4, 1, "ip", "float32"),
    (1, 2, 10, 1, 1, "mse", "float32"), (32, 1, 2049, 3, 3, "mse", "float32"),
    (256, 4, 1300, 8, 2, "mse", "float32"), (512, 3, 1100, 7, 1, "ip", "bfloat16"),
    (1000, 2, 1500, 5, 1, "mse", "float32")])
def test_attend_matches_oracle(d, bits, n, nqg, groups, mode, dtype):
    rng = np.random.default_rng(d * 11 + n)
    V = rng.standard_normal((groups * n, d)).astype(np.float32)
    L = (rng.standard_normal((groups * nqg, n)) * 3.0).astype(np.float32)
    if mode == "mse":
        plan, op = tq.tq_plan_create_mse(d, bits, 6), otq.make_mse_plan(d, bits, 6)
    else:
        plan, op = tq.tq_plan_create(d, bits, 6), otq.make_plan(d, bits, 6)
    vcodes = tq.tq_encode(plan, torch.from_numpy(V).to(DEV).to(getattr(torch, dtype)))
    logits = torch.from_numpy(L).to(DEV)
    out = tq.tq_attend(plan, logits, vcodes, n, 0.4, nq_per_group=nqg, n_groups=groups,
                       dtype=getattr(torch, dtype))
    torch.cuda.synchronize()
    c = vcodes.cpu().numpy()
    st = layout.unpack_mse(c, op.D, op.R) if mode == "mse" else layout.unpack(c, op.D, op.R)
    ref = otq.attend(op, L.astype(np.float64), dict(idx=st["idx"], norm=st["norm"]), 0.4, nqg)
    vmax = np.max(np.linalg.norm(otq.dequantize(op, st), axis=1))
    _check(_np(out), ref, vmax, dtype == "bfloat16", "attend d=%d n=%d" % (d, n))


def test_attend_with_logits_from_score():
    """The decode step as used: K codes scored (tq_score), then attention over V codes."""
    d, n, G, groups = 128, 3000, 4, 2
    rng = np.random.default_rng(2)
    K = torch.from_numpy(rng.standard_normal((groups * n, d)).astype(np.float32)).to(DEV)
    V = torch.from_numpy(rng.standard_normal((groups * n, d)).astype(np.float32)).to(DEV)
    Q = torch.from_numpy(rng.standard_normal((groups * G, d)).astype(np.float32)).to(DEV)
    kplan, vplan = tq.tq_plan_create(d, 3, 1), tq.tq_plan_create_mse(d, 3, 2)
    kc, vc = tq.tq_encode(kplan, K), tq.tq_encode(vplan, V)
    logits = tq.tq_score(kplan, Q, kc, n=n, nq_per_group=G, n_groups=groups)
    out = tq.tq_attend(vplan, logits, vc, n, 1.0 / np.sqrt(d), nq_per_group=G, n_groups=groups)
    torch.cuda.synchronize()
    op = otq.make_mse_plan(d, 3, 2)
    st = layout.unpack_mse(vc.cpu().numpy(), op.D, 3)
    ref = otq.attend(op, _np(logits), st, 1.0 / np.sqrt(d), G)
    vmax = np.max(np.linalg.norm(otq.dequantize(op, st), axis=1))
    _check(_np(out), ref, vmax, False, "score + attend")


def test_attend_uniform_logits_full_context_is_the_mean():
    """131072 tokens (128 chunks) with equal logits: the output is the mean of the
    dequantized values (computed from tq_dequantize), for every query row."""
    d, n = 128, 131072
    rng = np.random.default_rng(4)
    V = torch.from_numpy(rng.standard_normal((n, d)).astype(np.float32)).to(DEV)
    plan = tq.tq_plan_create_mse(d, 3, 0)
    vc = tq.tq_encode(plan, V)
    out = tq.tq_attend(plan, torch.full((4, n), 0.5, device=DEV), vc, n, 2.0)
    mean = tq.tq_dequantize(plan, vc, n).double().mean(0)
    torch.cuda.synchronize()
    assert torch.allclose(out.double(), mean.expand(4, d), rtol=0, atol=2e-5 * float(mean.norm()) + 1e-6)


def test_attend_rejects_split_plans_and_bad_sizes():
    m = np.zeros(64, dtype=np.uint8)
    m[:8] = 1
    plan = tq.tq_plan_create(64, 3, 0, m, 4)
    vc = torch.zeros((10, plan.record_bytes), dtype=torch.uint8, device=DEV)
    with pytest.raises(tq.TqError):
        tq.tq_attend(plan, torch.zeros((2, 10), device=DEV), vc, 10, 1.0)


@pytest.mark.parametrize("d,bits,n,nqg", [(128, 3, 4 * 1024 + 500, 4), (32, 1, 3 * 1024 + 100, 1),
                                          (64, 2, 2 * 1024 + 7, 6)])
def test_attend_many_groups_streams_several_chunks_per_workgroup(d, bits, n, nqg):
    """2048 groups: enough work that one workgroup streams several consecutive chunks (with
    the running max and norm scale carried across stages and reset per chunk); sampled groups
    against the oracle, the ragged last chunk included."""
    groups = 2048
    g = torch.Generator(device=DEV)
    g.manual_seed(d + n)
    V = torch.randn((groups * n, d), generator=g, device=DEV).to(torch.bfloat16)
    # a few large norms late in the sequence, so that the norm scale rises mid-chunk
    V[torch.arange(700, groups * n, 1537, device=DEV)] *= 40
    L = torch.randn((groups * nqg, n), generator=g, device=DEV) * 4
    L[:, 2000:2100] += 6          # the max of a row moves up in a later stage
    plan, op = tq.tq_plan_create_mse(d, bits, 3), otq.make_mse_plan(d, bits, 3)
    vc = tq.tq_encode(plan, V)
    out = tq.tq_attend(plan, L, vc, n, 0.7, nq_per_group=nqg, n_groups=groups)
    torch.cuda.synchronize()
    for grp in (0, 1, 1000, groups - 1):
        c = vc[grp * n:(grp + 1) * n].cpu().numpy()
        st = layout.unpack_mse(c, op.D, op.R)
        Lg = _np(L[grp * nqg:(grp + 1) * nqg])
        ref = otq.attend(op, Lg, st, 0.7, nqg)
        vmax = np.max(np.linalg.norm(otq.dequantize(op, st), axis=1))
        _check(_np(out[grp * nqg:(grp + 1) * nqg]), ref, vmax, False, "group %d" % grp)


def test_attend_zero_values_give_zero_rows():
    """Values that are all zero vectors (norm 0): every output row is exactly 0."""
    d, n = 128, 2500
    plan = tq.tq_plan_create_mse(d, 3, 1)
    vc = tq.tq_encode(plan, torch.zeros((n, d), device=DEV))
    L = torch.randn((4, n), device=DEV)
    out = tq.tq_attend(plan, L, vc, n, 1.0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("d,bits", [(32, 3), (32, 4), (64, 1), (512, 1), (512, 4), (1024, 4),
                                    (2048, 1), (2048, 4), (200, 1)])
def test_attend_every_index_width_on_each_kernel(d, bits):
    """Each (D, index bits) instantiation of both pass-1 kernels against the oracle, with 6
    query rows (two row quads where D <= 1024) and a ragged second chunk."""
    n, nqg = 1300, 6
    rng = np.random.default_rng(d * 7 + bits)
    V = rng.standard_normal((n, d)).astype(np.float32)
    L = (rng.standard_normal((nqg, n)) * 2.0).astype(np.float32)
    plan, op = tq.tq_plan_create_mse(d, bits, 4), otq.make_mse_plan(d, bits, 4)
    vc = tq.tq_encode(plan, torch.from_numpy(V).to(DEV))
    out = tq.tq_attend(plan, torch.from_numpy(L).to(DEV), vc, n, 0.5)
    torch.cuda.synchronize()
    st = layout.unpack_mse(vc.cpu().numpy(), op.D, op.R)
    ref = otq.attend(op, L.astype(np.float64), st, 0.5, nqg)
    vmax = np.max(np.linalg.norm(otq.dequantize(op, st), axis=1))
    _check(_np(out), ref, vmax, False, "attend d=%d bits=%d" % (d, bits))


@pytest.mark.parametrize("pattern", ["rising", "falling", "sharp", "very_negative"])
def test_attend_logit_patterns_that_move_the_reference(pattern):
    """Logits that climb across each chunk (the reference max moves by more than the slack
    many times), that fall (it never moves after the first stage), a large scale (most weights
    underflow to zero) and logits near -1e4 (only the differences matter)."""
    d, n, nqg, groups = 128, 2 * 1024 + 333, 4, 2
    rng = np.random.default_rng(len(pattern))
    V = rng.standard_normal((groups * n, d)).astype(np.float32)
    base = rng.standard_normal((groups * nqg, n))
    ramp = np.arange(n)[None, :] * 0.05
    scale = 1.0
    if pattern == "rising":
        L = base + ramp
    elif pattern == "falling":
        L = base - ramp
    elif pattern == "sharp":
        L, scale = base, 40.0
    else:
        L = base - 1e4
    L = L.astype(np.float32)
    plan, op = tq.tq_plan_create_mse(d, 3, 8), otq.make_mse_plan(d, 3, 8)
    vc = tq.tq_encode(plan, torch.from_numpy(V).to(DEV))
    out = tq.tq_attend(plan, torch.from_numpy(L).to(DEV), vc, n, scale, nq_per_group=nqg,
                       n_groups=groups)
    torch.cuda.synchronize()
    st = layout.unpack_mse(vc.cpu().numpy(), op.D, op.R)
    ref = otq.attend(op, L.astype(np.float64), st, scale, nqg)
    vmax = np.max(np.linalg.norm(otq.dequantize(op, st), axis=1))
    _check(_np(out), ref, vmax, False, "attend %s" % pattern)


@pytest.mark.parametrize("d,nqg", [(128, 4), (256, 8), (64, 16)])
def test_attend_masked_tokens(d, nqg):
    """-inf logits (masked tokens) weigh nothing: a row whose whole first chunk, or whole
    middle chunk, is masked, rows with scattered masks, and a masked tail; every row keeps at
    least one finite logit."""
    n, groups = 3 * 1024 + 200, 2
    rng = np.random.default_rng(d + nqg)
    V = rng.standard_normal((groups * n, d)).astype(np.float32)
    L = (rng.standard_normal((groups * nqg, n)) * 2.0).astype(np.float32)
    L[0, :1024] = -np.inf                  # first chunk masked
    L[1, 1024:2048] = -np.inf              # middle chunk masked
    L[2, rng.random(n) < 0.7] = -np.inf    # scattered
    L[3, 3 * 1024:] = -np.inf              # ragged tail masked
    L[nqg + 1, 1:] = -np.inf               # one visible token
    plan, op = tq.tq_plan_create_mse(d, 3, 8), otq.make_mse_plan(d, 3, 8)
    vc = tq.tq_encode(plan, torch.from_numpy(V).to(DEV))
    out = tq.tq_attend(plan, torch.from_numpy(L).to(DEV), vc, n, 0.7, nq_per_group=nqg,
                       n_groups=groups)
    torch.cuda.synchronize()
    st = layout.unpack_mse(vc.cpu().numpy(), op.D, op.R)
    ref = otq.attend(op, L.astype(np.float64), st, 0.7, nqg)
    assert np.all(np.isfinite(ref))
    vmax = np.max(np.linalg.norm(otq.dequantize(op, st), axis=1))
    _check(_np(out), ref, vmax, False, "attend masked d=%d" % d)
