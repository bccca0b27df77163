"""Layer plans (one outlier mask per head, shared tables; overview §4.1.1) through the C ABI:
one grouped encode and one score launch for all heads give, head by head, the codes and
scores of the per-head split plans, and match the oracle's split plan on that head's mask;
appends write straight into the cache rows."""
import numpy as np
import pytest

from oracle import turboquant as otq
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _masks(n_heads, d, n_out, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros((n_heads, d), dtype=np.uint8)
    for h in range(n_heads):
        m[h, rng.choice(d, n_out, replace=False)] = 1
    return m


def _keys(n_seq, n_heads, n, d, masks, seed):
    """[n_seq, n_heads, n, d] bf16 N(0,1) with each head's mask channels scaled x10."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_seq, n_heads, n, d)).astype(np.float32)
    x *= np.where(masks[None, :, None, :] == 1, 10.0, 1.0).astype(np.float32)
    return torch.from_numpy(x).to(DEV).to(torch.bfloat16)


@pytest.mark.parametrize("d,bits,obits,n_out", [(128, 3, 5, 32), (128, 2, 4, 32), (64, 3, 5, 16),
                                                (100, 4, 5, 25)])
def test_layer_plan_matches_per_head_plans_and_oracle(d, bits, obits, n_out):
    n_seq, n_heads, n, nqg = 2, 8, 777, 4
    masks = _masks(n_heads, d, n_out, d + bits)
    keys = _keys(n_seq, n_heads, n, d, masks, 7)
    groups = n_seq * n_heads
    rng = np.random.default_rng(8)
    q = torch.from_numpy(rng.standard_normal((groups * nqg, d)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    lp = tq.tq_plan_create_heads(d, bits, 5, masks, obits)
    assert lp.desc["n_heads"] == n_heads and lp.desc["n_subplans"] == 2
    codes = tq.tq_encode_groups(lp, keys.view(-1, d), groups)
    scores = tq.tq_score(lp, q, codes, n=n, nq_per_group=nqg, n_groups=groups)
    torch.cuda.synchronize()
    c = codes.view(n_seq, n_heads, n, -1)
    s = scores.view(n_seq, n_heads, nqg, n)
    for h in (0, 3, 7):
        hp = tq.tq_plan_create(d, bits, 5, masks[h], obits)
        assert hp.record_bytes == lp.record_bytes
        for sq in range(n_seq):
            ch = tq.tq_encode(hp, keys[sq, h])
            assert torch.equal(ch, c[sq, h]), "head %d seq %d records" % (h, sq)
            qh = q.view(n_seq, n_heads, nqg, d)[sq, h].contiguous()
            sh = tq.tq_score(hp, qh, ch, n=n)
            assert torch.equal(sh, s[sq, h]), "head %d seq %d scores" % (h, sq)
    # every (sequence, head) against the oracle's split plan on that head's mask; the
    # sub-plans' tables are the same for every head (only the channel lists differ), so the
    # code comparison pools all heads (the in-band mismatch budget is a fraction of them all)
    refs, gots = [[], []], [[], []]
    for h in range(n_heads):
        sp = otq.make_split_plan(d, bits, 5, masks[h], obits)
        for sq in range(n_seq):
            xs = keys[sq, h].float().cpu().numpy().astype(np.float64)
            ys = q.view(n_seq, n_heads, nqg, d)[sq, h].float().cpu().numpy().astype(np.float64)
            ref = otq.encode_split(sp, xs)
            got = parity.unpack_gpu(sp, c[sq, h].cpu().numpy())
            parity.check_scores_end_to_end(sp, ref, got, s[sq, h].cpu().numpy(), ys, xs,
                                           "layer plan head %d seq %d" % (h, sq))
            for i in range(2):
                refs[i].append(ref[i])
                gots[i].append(got[i])
    for i, p in enumerate(sp.plans):
        pooled_ref = {k: np.concatenate([r[k] for r in refs[i]]) for k in refs[i][0]}
        pooled_got = {k: np.concatenate([g[k] for g in gots[i]]) for k in gots[i][0]}
        parity.compare_codes(p, pooled_ref, pooled_got, "layer plan sub%d" % i)


def test_layer_plan_score_noalloc_and_topk():
    d, n_heads, n, nqg = 128, 4, 3000, 4
    masks = _masks(n_heads, d, 32, 11)
    keys = _keys(1, n_heads, n, d, masks, 12)
    lp = tq.tq_plan_create_heads(d, 3, 9, masks, 5)
    codes = tq.tq_encode_groups(lp, keys.view(-1, d), n_heads)
    q = torch.randn((n_heads * nqg, d), device=DEV).to(torch.bfloat16)
    ref = tq.tq_score(lp, q, codes, n=n, nq_per_group=nqg, n_groups=n_heads)
    out = torch.empty_like(ref)
    tq.tq_score_noalloc(lp, q, codes, n, out, nq_per_group=nqg, n_groups=n_heads)
    ids, vals = tq.tq_score_topk(lp, q, codes, n, 10, nq_per_group=nqg, n_groups=n_heads)
    ids2, vals2 = tq.tq_topk(ref, 10)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(ids, ids2) and torch.equal(vals, vals2)


def test_layer_plan_append_writes_cache_rows_directly():
    """One new key per (sequence, head) appended at the last slot of its group: the appended
    records equal tq_encode_groups of the same keys (one vector per group), rows outside the
    cache are skipped, every other row is untouched."""
    d, n_seq, n_heads, cap = 128, 3, 4, 50
    masks = _masks(n_heads, d, 32, 13)
    lp = tq.tq_plan_create_heads(d, 3, 4, masks, 5)
    groups = n_seq * n_heads
    cache = torch.randint(0, 256, (groups * cap, lp.record_bytes), dtype=torch.uint8, device=DEV)
    before = cache.clone()
    new = _keys(n_seq, n_heads, 1, d, masks, 14).view(groups, d)
    rows = torch.arange(groups, device=DEV, dtype=torch.int64) * cap + cap - 1
    rows[5] = groups * cap + 7          # outside the cache: skipped
    rows[6] = -1
    tq.tq_encode_scatter(lp, new, cache, rows)
    want = tq.tq_encode_groups(lp, new, groups)
    torch.cuda.synchronize()
    for i in range(groups):
        r = int(rows[i])
        if 0 <= r < groups * cap:
            assert torch.equal(cache[r], want[i]), "appended record %d" % i
    touched = torch.zeros(groups * cap, dtype=torch.bool, device=DEV)
    valid = (rows >= 0) & (rows < groups * cap)
    touched[rows[valid]] = True
    assert torch.equal(cache[~touched], before[~touched])


def test_layer_plan_invalid_calls():
    d = 64
    masks = _masks(4, d, 16, 15)
    lp = tq.tq_plan_create_heads(d, 3, 1, masks, 5)
    x = torch.randn((8, d), device=DEV).to(torch.bfloat16)
    with pytest.raises(tq.TqError):
        tq.tq_encode(lp, x)                      # rows need their head: tq_encode_groups
    codes = tq.tq_encode_groups(lp, x, 4)
    q = torch.randn((6, d), device=DEV).to(torch.bfloat16)
    with pytest.raises(tq.TqError):
        tq.tq_score(lp, q, codes, n=2, nq_per_group=2, n_groups=3)   # 3 groups, 4 heads
    bad = masks.copy()
    bad[1, np.flatnonzero(bad[1] == 0)[0]] = 1   # 17 outliers in head 1
    with pytest.raises(tq.TqError):
        tq.tq_plan_create_heads(d, 3, 1, bad, 5)
