"""Parity at the full benchmark sizes, in the launch configuration bench.py times,
on sampled outputs the oracle computes one by one."""
import numpy as np
import pytest

import workloads
from oracle import turboquant as otq
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_sampled(sp, codes_u8, x_rows, keys_idx, q_rows, scores_rows, tag):
    """codes of sampled keys vs the oracle; scores of the sampled (query, key) pairs, against
    the oracle's own codes where the codes are identical and the oracle on the GPU's codes
    elsewhere.  Returns the fraction of vectors with identical codes."""
    got = parity.unpack_gpu(sp, codes_u8)
    ref = otq.encode_split(sp, x_rows)
    for i, (p, r, g) in enumerate(zip(sp.plans, ref, got)):
        parity.compare_codes(p, r, g, "%s/sub%d" % (tag, i))
    return parity.check_scores_end_to_end(sp, ref, got, scores_rows, q_rows, x_rows, tag)


def test_kv_cache_shape_full():
    W = workloads.KV
    keys, queries, _ = workloads.kv_inputs(DEV, n_kv=W["n_kv"], n_tok=W["n_tok"], d=W["d"],
                                           group=W["group"], n_outlier=W["n_outlier"],
                                           outlier_scale=W["outlier_scale"], seed=W["seed"])
    n_kv, n_tok, d, G = W["n_kv"], W["n_tok"], W["d"], W["group"]
    plan = tq.tq_plan_create(d, W["bits"], W["seed"])
    sp = otq.make_split_plan(d, W["bits"], W["seed"])
    codes = tq.tq_encode(plan, keys.view(-1, d))
    scores = tq.tq_score(plan, queries, codes, n=n_tok, nq_per_group=G, n_groups=n_kv)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    for h in (0, 5, 7):
        kidx = np.sort(rng.choice(n_tok, 1024, replace=False))
        rows = h * n_tok + kidx
        frac = _check_sampled(sp, codes[torch.as_tensor(rows, device=DEV)].cpu().numpy(),
                              _np64(keys[h][torch.as_tensor(kidx, device=DEV)]), kidx,
                              _np64(queries[h * G:(h + 1) * G]),
                              scores[h * G:(h + 1) * G][:, torch.as_tensor(kidx, device=DEV)].cpu().numpy(),
                              "kv head %d" % h)
        assert frac > 0.99


@pytest.mark.parametrize("variant", ["3.5bit", "2.5bit"])
def test_split_shape_full(variant):
    W = workloads.SPLIT if variant == "3.5bit" else workloads.SPLIT_25
    keys, queries, ch = workloads.kv_inputs(DEV, n_kv=W["n_kv"], n_tok=W["n_tok"], d=W["d"],
                                            group=W["group"], n_outlier=W["n_outlier"],
                                            outlier_scale=W["outlier_scale"], seed=W["seed"])
    n_kv, n_tok, d, G = W["n_kv"], W["n_tok"], W["d"], W["group"]
    rng = np.random.default_rng(2)
    for h in range(n_kv):
        mask = np.zeros(d, dtype=np.uint8)
        mask[ch[h]] = 1
        plan = tq.tq_plan_create(d, W["bits"], W["seed"], mask, W["outlier_bits"])
        codes = tq.tq_encode(plan, keys[h])
        scores = tq.tq_score(plan, queries[h * G:(h + 1) * G], codes, n=n_tok)
        torch.cuda.synchronize()
        if h in (0, 3):
            sp = otq.make_split_plan(d, W["bits"], W["seed"], mask, W["outlier_bits"])
            kidx = np.sort(rng.choice(n_tok, 1024, replace=False))
            ki = torch.as_tensor(kidx, device=DEV)
            frac = _check_sampled(sp, codes[ki].cpu().numpy(), _np64(keys[h][ki]), kidx,
                                  _np64(queries[h * G:(h + 1) * G]), scores[:, ki].cpu().numpy(),
                                  "split %s head %d" % (variant, h))
            assert frac > 0.99


def test_long_context_shape_full_as_benchmarked():
    W = workloads.LONGCTX
    keys, queries, _ = workloads.longctx_inputs(DEV)
    n_seq, n_kv, n_tok, d, G = W["n_seq"], W["n_kv"], W["n_tok"], W["d"], W["group"]
    plan = tq.tq_plan_create(d, W["bits"], W["seed"])
    sp = otq.make_split_plan(d, W["bits"], W["seed"])
    codes = tq.tq_encode(plan, keys.view(-1, d))
    scores = tq.tq_score(plan, queries.view(-1, d), codes, n=n_tok, nq_per_group=G,
                         n_groups=n_seq * n_kv)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for (s, h) in ((0, 0), (7, 3), (15, 7)):
        kidx = np.sort(rng.choice(n_tok, 768, replace=False))
        ki = torch.as_tensor(kidx, device=DEV)
        g = s * n_kv + h
        rows = torch.as_tensor(g * n_tok + kidx, device=DEV)
        frac = _check_sampled(sp, codes[rows].cpu().numpy(), _np64(keys[s, h][ki]), kidx,
                              _np64(queries[s, h * G:(h + 1) * G]),
                              scores[g * G:(g + 1) * G][:, ki].cpu().numpy(),
                              "long-context seq %d head %d" % (s, h))
        assert frac > 0.99


def test_retrieval_shape_full_with_topk():
    W = workloads.RETRIEVAL
    keys, queries = workloads.retrieval_inputs(DEV, n_keys=W["n_keys"], n_queries=W["n_queries"],
                                               d=W["d"], seed=W["seed"])
    n, d, k = W["n_keys"], W["d"], W["topk"]
    plan = tq.tq_plan_create(d, W["bits"], W["seed"])
    sp = otq.make_split_plan(d, W["bits"], W["seed"])
    codes = tq.tq_encode(plan, keys)
    scores = tq.tq_score(plan, queries, codes, n=n)
    ids, vals = tq.tq_topk(scores, k)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    kidx = np.sort(rng.choice(n, 512, replace=False))
    qidx = np.sort(rng.choice(W["n_queries"], 8, replace=False))
    ki, qi = torch.as_tensor(kidx, device=DEV), torch.as_tensor(qidx, device=DEV)
    frac = _check_sampled(sp, codes[ki].cpu().numpy(), _np64(keys[ki]), kidx, _np64(queries[qi]),
                          scores[qi][:, ki].cpu().numpy(), "retrieval")
    assert frac > 0.99
    # top-k: values are the scores of the returned ids; the oracle's estimate of every
    # returned id is at least the oracle's estimate of any sampled key minus the tolerance
    ids_np, vals_np = ids.cpu().numpy(), vals.cpu().numpy()
    sc_rows = scores[qi].cpu().numpy()
    assert np.array_equal(vals_np[qidx], np.take_along_axis(sc_rows, ids_np[qidx], 1))
    assert np.all(np.diff(vals_np, axis=1) <= 0)
    for j, q in enumerate(qidx):
        cand = np.concatenate([ids_np[q], kidx])
        x = _np64(keys[torch.as_tensor(cand, device=DEV)])
        est = otq.score_split(sp, [parity.stored(c) for c in otq.encode_split(sp, x)],
                              _np64(queries[q:q + 1]))[0]
        qn = float(np.linalg.norm(_np64(queries[q])))
        kth = est[:k].min()
        assert np.all(est[k:] <= kth + 2e-3 * qn), "query %d: a sampled key beats the top-%d" % (q, k)
    # the fused call (as timed) returns exactly what score + top-k returned
    ids_f, vals_f = tq.tq_score_topk(plan, queries, codes, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(ids_f.cpu().numpy(), ids_np)
    assert np.array_equal(vals_f.cpu().numpy(), vals_np)
    # recall@10 of the estimate against exact fp32 inner products (reported)
    exact = queries[qi] @ keys.T
    top_exact = torch.topk(exact, k, dim=1).indices.cpu().numpy()
    recall = np.mean([len(set(top_exact[j]) & set(ids_np[q])) / k for j, q in enumerate(qidx)])
    print("recall@10 vs exact fp32 on %d queries: %.3f" % (len(qidx), recall))
    assert recall > 0.5


def test_mse_long_context_shape_full_as_benchmarked():
    """TurboQuant-MSE encode + dequantize of all 16.8 M long-context keys (the MSE bench
    step) and their scores against the 512 query heads (the MSE-key bench step); sampled
    records against the oracle's encode, their reconstructions against the oracle's
    dequantization of the stored codes, and sampled (query, key) scores against the oracle's
    quantized distance on the stored codes and, where the cells match, on its own codes."""
    from oracle import layout
    W = workloads.MSE_LONGCTX
    assert workloads.MSEKEYS_LONGCTX["bits"] == W["bits"] and workloads.MSEKEYS_LONGCTX["seed"] == W["seed"]
    keys, queries, _ = workloads.longctx_inputs(DEV)
    n_seq, n_kv, n_tok, d, G = W["n_seq"], W["n_kv"], W["n_tok"], W["d"], W["group"]
    plan = tq.tq_plan_create_mse(d, W["bits"], W["seed"])
    op = otq.make_mse_plan(d, W["bits"], W["seed"])
    flat = keys.view(-1, d)
    n = flat.shape[0]
    codes = tq.tq_encode(plan, flat)
    xh = tq.tq_dequantize(plan, codes, n, dtype=torch.bfloat16)
    scores = tq.tq_score(plan, queries.view(-1, d), codes, n=n_tok, nq_per_group=G,
                         n_groups=n_seq * n_kv)
    torch.cuda.synchronize()
    srng = np.random.default_rng(9)
    for (s, h) in ((0, 1), (9, 4), (15, 7)):
        kidx = np.sort(srng.choice(n_tok, 768, replace=False))
        ki = torch.as_tensor(kidx, device=DEV)
        g = s * n_kv + h
        rows = torch.as_tensor(g * n_tok + kidx, device=DEV)
        got = layout.unpack_mse(codes[rows].cpu().numpy(), op.D, W["bits"])
        x = _np64(keys[s, h][ki])
        own = otq.encode_mse(op, x)
        parity.compare_codes_mse(op, own, got, "mse keys seq %d head %d" % (s, h))
        y = _np64(queries[s, h * G:(h + 1) * G])
        est = scores[g * G:(g + 1) * G][:, ki].cpu().numpy().astype(np.float64)
        qn, xn = np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1)
        parity.check_scores(est, otq.score_mse(op, dict(idx=got["idx"], norm=got["norm"]), y),
                            qn, xn, "mse keys seq %d head %d" % (s, h))
        same = np.all(own["idx"] == got["idx"], axis=1)
        assert same.mean() > 0.99
        own_s = dict(idx=own["idx"][same], norm=own["norm"][same].astype(np.float32).astype(np.float64))
        parity.check_scores(est[:, same], otq.score_mse(op, own_s, y), qn, xn[same],
                            "mse keys seq %d head %d (oracle codes)" % (s, h))
    rng = np.random.default_rng(8)
    rows = np.sort(np.concatenate([rng.choice(n, 3000, replace=False), [0, n - 1]]))
    ri = torch.as_tensor(rows, device=DEV)
    got = layout.unpack_mse(codes[ri].cpu().numpy(), op.D, W["bits"])
    ref = otq.encode_mse(op, _np64(flat[ri]))
    parity.compare_codes_mse(op, ref, got, "mse long-context")
    xr = otq.dequantize(op, dict(idx=got["idx"], norm=got["norm"]))
    parity.check_dequantized(_np64(xh[ri]), xr, got["norm"], True, "mse long-context dequant")


def test_attend_long_context_shape_full_as_benchmarked():
    """Decode attention over the whole 16 x 8 x 131072 cache in the launch configuration the
    attend bench times (keys scored, values under the 3-bit MSE plan); sampled groups against
    the oracle's attention over the same logits and stored value codes."""
    import math
    from oracle import layout
    W = workloads.ATTEND_LONGCTX
    keys, queries, _ = workloads.longctx_inputs(DEV)
    vals, _, _ = workloads.longctx_inputs(DEV, seed=W["v_seed"])
    n_seq, n_kv, n_tok, d, G = W["n_seq"], W["n_kv"], W["n_tok"], W["d"], W["group"]
    n_groups = n_seq * n_kv
    kplan = tq.tq_plan_create(d, W["bits"], W["seed"])
    vplan = tq.tq_plan_create_mse(d, W["v_bits"], W["v_seed"])
    op = otq.make_mse_plan(d, W["v_bits"], W["v_seed"])
    kc = tq.tq_encode(kplan, keys.view(-1, d))
    vc = tq.tq_encode(vplan, vals.view(-1, d))
    del keys, vals
    logits = tq.tq_score(kplan, queries.view(-1, d), kc, n=n_tok, nq_per_group=G, n_groups=n_groups)
    out = tq.tq_attend(vplan, logits, vc, n_tok, 1.0 / math.sqrt(d), nq_per_group=G,
                       n_groups=n_groups, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for g in (0, 77, n_groups - 1):
        st = layout.unpack_mse(vc[g * n_tok:(g + 1) * n_tok].cpu().numpy(), op.D, op.R)
        L = logits[g * G:(g + 1) * G].double().cpu().numpy()
        ref = otq.attend(op, L, st, 1.0 / math.sqrt(d), G)
        got = out[g * G:(g + 1) * G].double().cpu().numpy()
        vmax = np.max(np.linalg.norm(otq.dequantize(op, st), axis=1))
        tol = 2e-5 * vmax + 2.0 ** -8 * np.abs(ref)
        assert np.all(np.abs(got - ref) <= tol), "group %d: max err/tol %g" % (g, np.max(np.abs(got - ref) / tol))
