"""Benchmark of the quantizer's hot path on one MI355X.

One step = encode every key of the long-context decode workload (norm split,
randomized Hadamard rotation, Lloyd-Max indices, QJL signs: one fused launch)
and score every query head against its KV head's codes (query preparation +
the streaming estimator).  Inputs are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--copy-calibration MIB] [--workload NAME]

`--workload` selects one of the other synthetic shapes (kv, split35, split25,
retrieval, retrieval2, small, mse, attend, decode); their step is encode + score (+ top-k for
`small`; one fused score + top-k call for `retrieval`, whose roofline is the
MFMA one; `retrieval2` adds the exact re-rank of a quantized top-64; for `mse`,
TurboQuant-MSE encode + dequantize of the long-context keys, counted in
vectors/s; `attend` is one decode step over the long-context cache held
quantized, keys scored and values attended, counted in (query, token) pairs/s;
`decode` is the whole decode step over that cache, one token per head appended
to both caches, then scoring and attention, counted in steps/s) and the line carries the same fields, without the CPU leg; the two retrieval
lines also report recall@10 against an exact fp32 search.

Prints one JSON line.  `value` is scores per second over whole steps; the
per-kernel rates, the roofline of the dominant kernel (algorithmic bytes per
launch / mean HIP-event duration on the launch stream) and the fp64 CPU oracle
timed on a bounded sample of the same workload ride along.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_16BIT_TFLOPS = 2500.0     # dense bf16 and fp16 matrix peak of the MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-groups", type=int, default=16)
    ap.add_argument("--workload", default="longctx",
                    choices=["longctx", "kv", "split35", "split25", "retrieval", "retrieval2",
                             "small", "mse", "attend", "decode", "msekeys", "retrievalmse",
                             "decodemse"],
                    help="long-context decode (default, the headline line); the other shapes "
                         "report the same fields for their own step (no CPU leg)")
    ap.add_argument("--hbm-rotate", type=int, default=0, metavar="MIB",
                    help="kv, split35, split25: keep copies of a step's inputs and outputs "
                         "filling MIB MiB and use the next copy each step, so that every step "
                         "reads HBM rather than the 256 MB Infinity Cache")
    ap.add_argument("--no-hbm-ceiling", action="store_true",
                    help="skip the plain copy / read of 2 GiB measured after the timed steps")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB three times (untimed), so a "
                         "counter run can scale its byte counters by a copy of known size")
    return ap.parse_args()


KERNEL_DIR = os.path.join(ROOT, "rotation_online_vector_amd", "csrc")

# the arithmetic of each workload's step, by the operand formats its kernels use
MIXED_D128 = "f16+f8+f4 mfma, f32 acc"
DTYPES = {
    "longctx": MIXED_D128, "kv": MIXED_D128, "split35": MIXED_D128, "split25": MIXED_D128,
    "small": "bf16+f8+f4 mfma, f32 acc", "attend": MIXED_D128 + "; fp16 mfma attention",
    "decode": MIXED_D128 + "; fp16 mfma attention", "mse": "fp16 mfma, f32 acc",
    "retrieval": "f32 fwht; bf16 mfma signs and query projection; fp16 mfma scores; f32 acc",
    "retrieval2": "f32 fwht; bf16 mfma signs and query projection; fp16 mfma scores; f32 acc",
    "msekeys": "fp16 mfma rotation (encode); f8+f4 mfma scores; f32 acc",
    "decodemse": "f8+f4 mfma scores; fp16 mfma attention; f32 acc",
    "retrievalmse": "f32 fwht; fp16 mfma scores; f32 acc",
}
OPERANDS_D128 = {
    "tq_encode": "bf16 keys scaled to fp16 against the exact integer rotation in fp16; the "
                 "residual as an fp16 limb against 2^8 S in fp16 plus an fp8 e4m3 limb against "
                 "S in e4m3; fp32 accumulation, norms and comparisons",
    "tq_score": "the rotated query and its QJL projection as three fp8 e4m3 limbs against "
                "the key bit planes as fp4 {0, 1/2}; fp32 accumulation and epilogue",
}


def kernel_sources_sha256(files):
    """sha256 over the named kernel sources (files of the library's csrc/), in the given
    order: a stored counter record names the sources of the kernels it measured."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(KERNEL_DIR, f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload, kernel_key):
    """HBM bytes per launch of entry point `kernel_key` on `workload` from the stored counter
    runs (profiles/traffic_<workload>.json: FETCH_SIZE and WRITE_SIZE scaled by a copy of known
    size), or None when there is no record or the sources of the measured kernels (listed in
    the record) changed since the counters were taken."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)))
        k = rec.get("kernels", {}).get(kernel_key)
        if k is None or kernel_sources_sha256(k["sources"]) != k.get("sources_sha256"):
            return None
    except (OSError, ValueError, KeyError, TypeError):
        return None
    return k.get("hbm_bytes")


def cpu_baseline(keys, queries, group, bits, seed, n_groups):
    """The fp64 oracle, as it stands, on the first `n_groups` (sequence, KV head) groups:
    encode all their keys and score them against their query heads (same work per key as
    one step of the GPU path)."""
    import numpy as np
    from oracle import turboquant as otq
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    n_seq, n_kv, n_tok, d = keys.shape
    plan = otq.make_plan(d, bits, seed)
    n_scores, n_keys, dt_enc, dt_sc = 0, 0, 0.0, 0.0
    for g in range(n_groups):
        s, h = divmod(g, n_kv)
        x = keys[s, h].float().cpu().numpy().astype(np.float64)
        y = queries[s, h * group:(h + 1) * group].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        codes = otq.encode(plan, x)
        t1 = time.perf_counter()
        est = otq.score(plan, codes, y)
        dt_enc += t1 - t0
        dt_sc += time.perf_counter() - t1
        n_scores += est.size
        n_keys += x.shape[0]
    dt = dt_enc + dt_sc
    return {"value": n_scores / dt, "unit": "scores/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "encode_vectors_per_s": n_keys / dt_enc, "score_scores_per_s": n_scores / dt_sc,
            "sample": "%d of %d (sequence, KV head) groups: %d keys encoded and scored against "
                      "their %d query heads in fp64 (plan solve excluded), %.1f s of CPU time"
                      % (n_groups, n_seq * n_kv, n_groups * n_tok, group, dt)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def hbm_ceiling(dev, mib=2048, reps=5):
    """What a plain streaming kernel reaches on this device, next to the 8 TB/s nominal: a
    device-to-device copy of `mib` MiB (the runtime's copy kernel), bytes read + written,
    mean of `reps` runs, measured after the timed steps."""
    import torch
    nb = mib << 20
    src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    out = {}
    for name, fn, moved in (("copy_gbs", lambda: dst.copy_(src), 2 * nb),):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[name] = round(moved * reps / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    out["note"] = "device copy of %d MiB (read + write), mean of %d" % (mib, reps)
    del src, dst
    return out


def _rate(n, ms):
    return n / ms * 1e3 if ms > 0 else None


def _copies(rotate_mib, set_bytes):
    """Number of copies of a step's buffers that fill rotate_mib MiB (1: no rotation)."""
    if rotate_mib <= 0:
        return 1
    return max(2, -(-(rotate_mib << 20) // set_bytes))


def build_workload(name, dev, W_all, rotate_mib=0):
    """Inputs resident on the device, plans, output buffers and the launch phases of one step.

    Returns dict(config, phases=[(entry point, fn)], bytes={entry point: algorithmic bytes},
    n_keys, n_scores, keep) -- each fn enqueues that entry point's launches for one step."""
    import torch
    import rotation_online_vector_amd as tq
    import workloads
    W = W_all[name]
    if name in ("longctx", "msekeys"):
        keys, queries, _ = workloads.longctx_inputs(dev)
        n_seq, n_kv, n_tok, d, G = W["n_seq"], W["n_kv"], W["n_tok"], W["d"], W["group"]
        n_keys, n_groups = n_seq * n_kv * n_tok, n_seq * n_kv
        plan = (tq.tq_plan_create_mse if name == "msekeys" else tq.tq_plan_create)(
            d, W["bits"], W["seed"])
        rb = plan.record_bytes
        codes = torch.empty((n_keys, rb), dtype=torch.uint8, device=dev)
        scores = torch.empty((n_groups * G, n_tok), dtype=torch.float32, device=dev)
        xk, qv = keys.view(n_keys, d), queries.view(n_groups * G, d)
        n_scores = n_groups * G * n_tok
        return dict(
            config={"workload": W["name"], "n_seq": n_seq, "kv_heads": n_kv, "tokens": n_tok,
                    "d": d, "bits": W["bits"], "query_heads_per_seq": n_kv * G, "gqa_group": G,
                    "keys_per_step": n_keys, "scores_per_step": n_scores, "record_bytes": rb,
                    **({"mode": "mse"} if name == "msekeys" else {})},
            phases=[("tq_encode", lambda: tq.tq_encode(plan, xk, codes)),
                    ("tq_score", lambda: tq.tq_score(plan, qv, codes, n=n_tok, nq_per_group=G,
                                                     n_groups=n_groups, scores=scores))],
            bytes={"tq_encode": n_keys * d * 2 + n_keys * rb,
                   "tq_score": n_keys * rb + n_scores * 4 + n_groups * G * d * 2},
            n_keys=n_keys, n_scores=n_scores,
            keep=(plan, keys, queries, codes, scores))
    if name == "mse":
        keys, _, _ = workloads.longctx_inputs(dev)
        n_seq, n_kv, n_tok, d = W["n_seq"], W["n_kv"], W["n_tok"], W["d"]
        n_keys = n_seq * n_kv * n_tok
        plan = tq.tq_plan_create_mse(d, W["bits"], W["seed"])
        rb = plan.record_bytes
        codes = torch.empty((n_keys, rb), dtype=torch.uint8, device=dev)
        xh = torch.empty((n_keys, d), dtype=torch.bfloat16, device=dev)
        xk = keys.view(n_keys, d)
        return dict(
            config={"workload": W["name"], "n_seq": n_seq, "kv_heads": n_kv, "tokens": n_tok,
                    "d": d, "bits": W["bits"], "mode": "mse", "keys_per_step": n_keys,
                    "record_bytes": rb},
            phases=[("tq_encode", lambda: tq.tq_encode(plan, xk, codes)),
                    ("tq_dequantize", lambda: tq.tq_dequantize(plan, codes, n_keys, x=xh))],
            bytes={"tq_encode": n_keys * d * 2 + n_keys * rb,
                   "tq_dequantize": n_keys * rb + n_keys * d * 2},
            n_keys=n_keys, n_scores=None,
            value=(n_keys, "vectors/s",
                   "TurboQuant-MSE encode + dequantize vectors/sec (d=128, 3-bit)"),
            keep=(plan, keys, codes, xh))
    if name in ("decode", "decodemse"):
        keys, queries, _ = workloads.longctx_inputs(dev)
        vals, _, _ = workloads.longctx_inputs(dev, seed=W["v_seed"])
        n_seq, n_kv, n_tok, d, G = W["n_seq"], W["n_kv"], W["n_tok"], W["d"], W["group"]
        n_keys, n_groups = n_seq * n_kv * n_tok, n_seq * n_kv
        # decodemse: the keys too under the 3-bit MSE plan (overview §4.1.1, most heads)
        kplan = (tq.tq_plan_create_mse if name == "decodemse" else tq.tq_plan_create)(
            d, W["bits"], W["seed"])
        vplan = tq.tq_plan_create_mse(d, W["v_bits"], W["v_seed"])
        kcodes = tq.tq_encode(kplan, keys.view(n_keys, d))
        vcodes = tq.tq_encode(vplan, vals.view(n_keys, d))
        # the step's new tokens: row n_tok - 1 of every group, appended in place
        gidx = torch.arange(n_groups, device=dev, dtype=torch.int64) * n_tok + (n_tok - 1)
        new_k = keys.view(n_keys, d)[gidx].clone()
        new_v = vals.view(n_keys, d)[gidx].clone()
        del keys, vals
        rows = n_groups * G
        logits = torch.empty((rows, n_tok), dtype=torch.float32, device=dev)
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=dev)
        qv = queries.view(rows, d)
        n_scores = rows * n_tok
        krb, vrb = kplan.record_bytes, vplan.record_bytes

        def append():
            tq.tq_encode_scatter(kplan, new_k, kcodes, gidx)
            tq.tq_encode_scatter(vplan, new_v, vcodes, gidx)
        return dict(
            config={"workload": W["name"], "n_seq": n_seq, "kv_heads": n_kv, "tokens": n_tok,
                    "d": d, "k_bits": W["bits"], "v_bits": W["v_bits"], "v_mode": "mse",
                    "k_mode": "mse" if name == "decodemse" else "inner_product",
                    "query_heads_per_seq": n_kv * G, "gqa_group": G, "keys_per_step": n_groups,
                    "scores_per_step": n_scores, "record_bytes": krb + vrb,
                    "k_record_bytes": krb, "v_record_bytes": vrb, "cache_tokens": n_keys,
                    "cache_bytes": n_keys * (krb + vrb),
                    "append": "one token per (sequence, KV head) to both caches per step"},
            phases=[("tq_encode_scatter", append),
                    ("tq_score", lambda: tq.tq_score(kplan, qv, kcodes, n=n_tok, nq_per_group=G,
                                                     n_groups=n_groups, scores=logits)),
                    ("tq_attend", lambda: tq.tq_attend(vplan, logits, vcodes, n_tok,
                                                       1.0 / math.sqrt(d), nq_per_group=G,
                                                       n_groups=n_groups, out=out))],
            bytes={"tq_encode_scatter": n_groups * (4 * d + krb + vrb + 16),
                   "tq_score": n_keys * krb + n_scores * 4 + rows * d * 2,
                   "tq_attend": n_keys * vrb + n_scores * 4 + rows * d * 2},
            n_keys=n_groups, n_scores=n_scores,
            value=(1, "steps/s",
                   "decode steps/sec over a quantized KV cache (d=128, 16x8x131072 tokens: "
                   "append 1 token per head, score 3-bit keys, attend 3-bit MSE values)"),
            keep=(kplan, vplan, queries, kcodes, vcodes, logits, out, new_k, new_v, gidx))
    if name == "attend":
        keys, queries, _ = workloads.longctx_inputs(dev)
        vals, _, _ = workloads.longctx_inputs(dev, seed=W["v_seed"])
        n_seq, n_kv, n_tok, d, G = W["n_seq"], W["n_kv"], W["n_tok"], W["d"], W["group"]
        n_keys, n_groups = n_seq * n_kv * n_tok, n_seq * n_kv
        kplan = tq.tq_plan_create(d, W["bits"], W["seed"])
        vplan = tq.tq_plan_create_mse(d, W["v_bits"], W["v_seed"])
        kcodes = tq.tq_encode(kplan, keys.view(n_keys, d))
        vcodes = tq.tq_encode(vplan, vals.view(n_keys, d))
        del keys, vals
        rows = n_groups * G
        logits = torch.empty((rows, n_tok), dtype=torch.float32, device=dev)
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=dev)
        qv = queries.view(rows, d)
        n_scores = rows * n_tok
        krb, vrb = kplan.record_bytes, vplan.record_bytes
        return dict(
            config={"workload": W["name"], "n_seq": n_seq, "kv_heads": n_kv, "tokens": n_tok,
                    "d": d, "k_bits": W["bits"], "v_bits": W["v_bits"], "v_mode": "mse",
                    "query_heads_per_seq": n_kv * G, "gqa_group": G, "keys_per_step": n_keys,
                    "scores_per_step": n_scores, "record_bytes": krb + vrb,
                    "k_record_bytes": krb, "v_record_bytes": vrb,
                    "cache": "encoded before the timed steps (a decode step reads it)"},
            phases=[("tq_score", lambda: tq.tq_score(kplan, qv, kcodes, n=n_tok, nq_per_group=G,
                                                     n_groups=n_groups, scores=logits)),
                    ("tq_attend", lambda: tq.tq_attend(vplan, logits, vcodes, n_tok,
                                                       1.0 / math.sqrt(d), nq_per_group=G,
                                                       n_groups=n_groups, out=out))],
            bytes={"tq_score": n_keys * krb + n_scores * 4 + rows * d * 2,
                   "tq_attend": n_keys * vrb + n_scores * 4 + rows * d * 2},
            n_keys=n_keys, n_scores=n_scores,
            value=(n_scores, "pairs/s",
                   "decode attention over a quantized KV cache: (query, token) pairs/sec "
                   "(d=128, 3-bit keys scored, 3-bit MSE values attended)"),
            keep=(kplan, vplan, queries, kcodes, vcodes, logits, out))
    if name == "kv":
        keys, queries, _ = workloads.kv_inputs(dev, n_kv=W["n_kv"], n_tok=W["n_tok"], d=W["d"],
                                               group=W["group"], n_outlier=W["n_outlier"],
                                               outlier_scale=W["outlier_scale"], seed=W["seed"])
        n_kv, n_tok, d, G = W["n_kv"], W["n_tok"], W["d"], W["group"]
        n_keys = n_kv * n_tok
        plan = tq.tq_plan_create(d, W["bits"], W["seed"])
        rb = plan.record_bytes
        codes = torch.empty((n_keys, rb), dtype=torch.uint8, device=dev)
        scores = torch.empty((n_kv * G, n_tok), dtype=torch.float32, device=dev)
        xk = keys.view(n_keys, d)
        n_scores = n_kv * G * n_tok
        R = _copies(rotate_mib, n_keys * d * 2 + n_keys * rb + n_scores * 4)
        xs = [xk] + [xk.clone() for _ in range(R - 1)]
        cs = [codes] + [torch.empty_like(codes) for _ in range(R - 1)]
        ss = [scores] + [torch.empty_like(scores) for _ in range(R - 1)]
        cur = [0]
        return dict(
            config={"workload": W["name"], "kv_heads": n_kv, "tokens": n_tok, "d": d,
                    "bits": W["bits"], "gqa_group": G, "keys_per_step": n_keys,
                    "scores_per_step": n_scores, "record_bytes": rb},
            phases=[("tq_encode", lambda: tq.tq_encode(plan, xs[cur[0]], cs[cur[0]])),
                    ("tq_score", lambda: tq.tq_score(plan, queries, cs[cur[0]], n=n_tok,
                                                     nq_per_group=G, n_groups=n_kv,
                                                     scores=ss[cur[0]]))],
            bytes={"tq_encode": n_keys * d * 2 + n_keys * rb,
                   "tq_score": n_keys * rb + n_scores * 4 + n_kv * G * d * 2},
            copies=R, advance=lambda: cur.__setitem__(0, (cur[0] + 1) % R),
            n_keys=n_keys, n_scores=n_scores, keep=(plan, keys, queries, xs, cs, ss))
    if name in ("split35", "split25"):
        import numpy as np
        keys, queries, ch = workloads.kv_inputs(dev, n_kv=W["n_kv"], n_tok=W["n_tok"], d=W["d"],
                                                group=W["group"], n_outlier=W["n_outlier"],
                                                outlier_scale=W["outlier_scale"], seed=W["seed"])
        n_kv, n_tok, d, G = W["n_kv"], W["n_tok"], W["d"], W["group"]
        # one layer plan: each head's own outlier mask, shared tables; one grouped encode
        # and one score call cover all heads
        masks = np.zeros((n_kv, d), dtype=np.uint8)
        for h in range(n_kv):
            masks[h, ch[h]] = 1
        plan = tq.tq_plan_create_heads(d, W["bits"], W["seed"], masks, W["outlier_bits"])
        rb = plan.record_bytes
        codes = torch.empty((n_kv * n_tok, rb), dtype=torch.uint8, device=dev)
        scores = torch.empty((n_kv * G, n_tok), dtype=torch.float32, device=dev)
        xk, qv = keys.view(n_kv * n_tok, d), queries.view(n_kv * G, d)
        R = _copies(rotate_mib, n_kv * n_tok * (d * 2 + rb) + n_kv * G * n_tok * 4)
        xs = [xk] + [xk.clone() for _ in range(R - 1)]
        cs = [codes] + [torch.empty_like(codes) for _ in range(R - 1)]
        ss = [scores] + [torch.empty_like(scores) for _ in range(R - 1)]
        cur = [0]

        def enc():
            tq.tq_encode_groups(plan, xs[cur[0]], n_kv, cs[cur[0]])

        def sco():
            tq.tq_score(plan, qv, cs[cur[0]], n=n_tok, nq_per_group=G, n_groups=n_kv,
                        scores=ss[cur[0]])
        n_keys, n_scores = n_kv * n_tok, n_kv * G * n_tok
        return dict(
            config={"workload": W["name"], "kv_heads": n_kv, "tokens": n_tok, "d": d,
                    "bits": W["bits"], "outlier_bits": W["outlier_bits"],
                    "outlier_channels": W["n_outlier"], "gqa_group": G, "keys_per_step": n_keys,
                    "scores_per_step": n_scores, "record_bytes": rb},
            phases=[("tq_encode", enc), ("tq_score", sco)],
            bytes={"tq_encode": n_keys * d * 2 + n_keys * rb,
                   "tq_score": n_keys * rb + n_scores * 4 + n_kv * G * d * 2},
            copies=R, advance=lambda: cur.__setitem__(0, (cur[0] + 1) % R),
            n_keys=n_keys, n_scores=n_scores, keep=(plan, keys, queries, xs, cs, ss))
    if name in ("retrieval", "retrieval2", "small", "retrievalmse"):
        if name != "small":
            keys, queries = workloads.retrieval_inputs(dev, n_keys=W["n_keys"],
                                                       n_queries=W["n_queries"], d=W["d"],
                                                       seed=W["seed"])
        else:
            k_np, q_np = workloads.small_inputs(W["n_keys"], W["n_queries"], W["d"], W["seed"])
            keys, queries = torch.from_numpy(k_np).to(dev), torch.from_numpy(q_np).to(dev)
        n, nq, d, k = W["n_keys"], W["n_queries"], W["d"], W.get("topk", 10)
        plan = (tq.tq_plan_create_mse if name == "retrievalmse" else tq.tq_plan_create)(
            d, W["bits"], W["seed"])
        rb = plan.record_bytes
        D = plan.desc["sub"][0]["D"]
        codes = torch.empty((n, rb), dtype=torch.uint8, device=dev)
        ids = torch.empty((nq, k), dtype=torch.int64, device=dev)
        vals = torch.empty((nq, k), dtype=torch.float32, device=dev)
        config = {"workload": W["name"], "keys": n, "queries": nq, "d": d, "D": D,
                  "bits": W["bits"], "topk": k, "keys_per_step": n, "scores_per_step": n * nq,
                  "record_bytes": rb, **({"mode": "mse"} if name == "retrievalmse" else {})}
        enc = ("tq_encode", lambda: tq.tq_encode(plan, keys, codes))
        enc_bytes = n * d * 4 + n * rb
        def recall_at_k(ids_fn, sample=64):
            """recall@k of the step's ids against an exact fp32 search, on the first
            `sample` queries (measured after the timed steps)."""
            def run():
                got = ids_fn()[:sample].cpu().numpy()
                exact = torch.topk(queries[:sample] @ keys.T, k, dim=1).indices.cpu().numpy()
                r = float(np.mean([len(set(exact[q]) & set(got[q].tolist())) / k
                                   for q in range(len(got))]))
                return {"recall_at_%d" % k: round(r, 4), "queries_sampled": len(got),
                        "against": "exact fp32 inner products over all keys"}
            return run
        import numpy as np
        if name == "retrieval2":
            # two-stage retrieval: quantized top-64, then the exact top-k of those 64
            kc = 64
            cand = torch.empty((nq, kc), dtype=torch.int64, device=dev)
            cvals = torch.empty((nq, kc), dtype=torch.float32, device=dev)
            return dict(
                config=dict(config, candidates=kc),
                phases=[enc, ("tq_score_topk",
                              lambda: tq.tq_score_topk(plan, queries, codes, n, kc, ids=cand, vals=cvals)),
                        ("tq_rerank", lambda: tq.tq_rerank(queries, keys, cand, k, ids=ids, vals=vals))],
                bytes={"tq_encode": enc_bytes, "tq_score_topk": n * rb + nq * d * 4 + nq * kc * 12,
                       "tq_rerank": nq * kc * (8 + d * 4) + nq * d * 4 + nq * k * 12},
                flops={"tq_encode": 2.0 * D * D * n, "tq_score_topk": 2.0 * (2 * D) * n * nq,
                       "tq_rerank": 2.0 * d * kc * nq},
                quality=recall_at_k(lambda: ids),
                n_keys=n, n_scores=n * nq, keep=(plan, keys, queries, codes, ids, vals, cand, cvals))
        if name == "retrievalmse":
            # an MSE index (overview §4.2.1) searched by the quantized distance (§4.2.2): the
            # scores go to the per-stream workspace and the top-k is selected from them
            return dict(
                config=config,
                phases=[enc, ("tq_score_topk",
                              lambda: tq.tq_score_topk(plan, queries, codes, n, k, ids=ids, vals=vals))],
                bytes={"tq_encode": enc_bytes, "tq_score_topk": n * rb + nq * d * 4 + nq * k * 12},
                # MFMA work: the centroid terms of every (query, key) pair (2 D per score)
                flops={"tq_score_topk": 2.0 * D * n * nq},
                quality=recall_at_k(lambda: ids),
                n_keys=n, n_scores=n * nq, keep=(plan, keys, queries, codes, ids, vals))
        if name == "retrieval":
            # score and select in one call: the score matrix is never stored
            return dict(
                config=config,
                phases=[enc, ("tq_score_topk",
                              lambda: tq.tq_score_topk(plan, queries, codes, n, k, ids=ids, vals=vals))],
                bytes={"tq_encode": enc_bytes, "tq_score_topk": n * rb + nq * d * 4 + nq * k * 12},
                # MFMA work: the sign projection (2 k D per key, k = D) and the bit-sliced
                # scorer's contraction of every key with every query (2 (D + k) per score)
                flops={"tq_encode": 2.0 * D * D * n, "tq_score_topk": 2.0 * (2 * D) * n * nq},
                quality=recall_at_k(lambda: ids),
                n_keys=n, n_scores=n * nq, keep=(plan, keys, queries, codes, ids, vals))
        scores = torch.empty((nq, n), dtype=torch.float32, device=dev)
        return dict(
            config=config,
            phases=[enc, ("tq_score", lambda: tq.tq_score(plan, queries, codes, n=n, scores=scores)),
                    ("tq_topk", lambda: tq.tq_topk(scores, k, ids, vals))],
            bytes={"tq_encode": enc_bytes, "tq_score": n * rb + n * nq * 4 + nq * d * 4,
                   "tq_topk": n * nq * 4 + nq * k * 12},
            n_keys=n, n_scores=n * nq, keep=(plan, keys, queries, codes, scores, ids, vals))
    raise ValueError(name)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only; --gpus %d is not supported (the multi-GPU layout "
              "is described in DESIGN.md, not run)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import workloads

    W_all = {"longctx": workloads.LONGCTX, "kv": workloads.KV, "split35": workloads.SPLIT,
             "split25": workloads.SPLIT_25, "retrieval": workloads.RETRIEVAL,
             "small": workloads.SMALL, "mse": workloads.MSE_LONGCTX,
             "attend": workloads.ATTEND_LONGCTX, "decode": workloads.DECODE_LONGCTX,
             "retrieval2": dict(workloads.RETRIEVAL, name=workloads.RETRIEVAL["name"] + "-2stage"),
             "msekeys": workloads.MSEKEYS_LONGCTX, "retrievalmse": workloads.RETRIEVAL_MSE,
             "decodemse": workloads.DECODE_MSE_LONGCTX}
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.hbm_rotate and args.workload not in ("kv", "split35", "split25"):
        print("--hbm-rotate applies to kv, split35 and split25 (the others exceed the cache)",
              file=sys.stderr)
        sys.exit(2)
    wl = build_workload(args.workload, dev, W_all, args.hbm_rotate)
    # the code set of the smaller shapes fits the 256 MB Infinity Cache: their GB/s are
    # cache-resident effective rates, not HBM rates
    code_bytes = wl["config"].get("cache_bytes",
                                  wl["config"]["keys_per_step"] * wl["config"]["record_bytes"])
    n_value, unit, metric = wl.get("value") or (
        wl["n_scores"], "scores/s",
        "quantized-key scores/sec + HBM GB/s (d=128, 3-bit); encode vectors/sec")
    wl["config"]["residency"] = (
        ("cache-resident: %.0f MB of codes, under the 256 MB Infinity Cache (effective GB/s)"
         if code_bytes < 256e6 else "HBM: %.0f MB of codes") % (code_bytes / 1e6))
    if wl.get("copies", 1) > 1:
        wl["config"]["residency"] = (
            "HBM, buffer-rotated: %d copies of the step's inputs and outputs (%.0f MB of codes "
            "each), the next copy every step" % (wl["copies"], code_bytes / 1e6))
        wl["config"]["buffer_copies"] = wl["copies"]
    phases = wl["phases"]
    stream = torch.cuda.current_stream()

    advance = wl.get("advance")

    def step(ev=None):
        if advance is not None:
            advance()
        for i, (_, fn) in enumerate(phases):
            if ev is not None:
                ev[i].record(stream)
            fn()
        if ev is not None:
            ev[len(phases)].record(stream)

    if args.copy_calibration > 0:
        nb = args.copy_calibration << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    kern = {}
    for i, (nm, _) in enumerate(phases):
        t = np.array([e[i].elapsed_time(e[i + 1]) for e in evs])
        ms = float(np.mean(t))
        b = wl["bytes"][nm]
        kern[nm] = {"ms": ms, "bytes": b, "gbs": b / ms / 1e6,
                    "pct": [float(x) for x in np.percentile(t, [10, 50, 90])]}
    ceiling = hbm_ceiling(dev) if not args.no_hbm_ceiling else None
    dom = max(kern, key=lambda k: kern[k]["ms"])
    flops = wl.get("flops")
    for k, v in kern.items():
        if flops and k in flops:
            v["tflops"] = flops[k] / (v["ms"] * 1e-3) / 1e12
    if flops and dom in flops:
        # a contraction-bound workload: algorithmic MFMA flops per launch against the dense
        # 16-bit peak (the sign projection runs on bf16 MFMA, the scorer on fp16: one peak)
        tf = kern[dom]["tflops"]
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_16BIT_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / MFMA_16BIT_TFLOPS, 4), "traffic": None,
                "flops_per_launch": flops[dom]}
    else:
        # the decode step runs the attention workload's kernels on the same cache
        traffic = measured_traffic("attend" if args.workload in ("decode", "decodemse") else args.workload, dom)
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(kern[dom]["gbs"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kern[dom]["gbs"] / HBM_PEAK_GBS, 4),
                "traffic": traffic, "bytes_per_launch": kern[dom]["bytes"]}
    score_key = "tq_score" if "tq_score" in kern else (
        "tq_score_topk" if "tq_score_topk" in kern else None)
    out = {
        "metric": metric,
        "value": n_value / (ms_step / 1e3),
        "unit": unit,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPES[args.workload], "data": "synthetic",
        "config": wl["config"],
        "encode_vectors_per_s": (_rate(wl["n_keys"], kern["tq_encode"]["ms"])
                                 if "tq_encode" in kern else None),
        "score_scores_per_s": _rate(wl["n_scores"], kern[score_key]["ms"]) if score_key else None,
        "kernels": {k: dict({"ms": round(v["ms"], 4),
                             "ms_p10_p50_p90": [round(x, 4) for x in v["pct"]],
                             "alg_bytes": v["bytes"],
                             "alg_gbs": round(v["gbs"], 1),
                             "hbm_frac": round(v["gbs"] / HBM_PEAK_GBS, 4)},
                            **({"mfma_tflops": round(v["tflops"], 1),
                                "mfma_frac": round(v["tflops"] / MFMA_16BIT_TFLOPS, 4)}
                               if "tflops" in v else {}))
                    for k, v in kern.items()},
        "roofline": roof,
        "hbm_ceiling": ceiling,
    }
    if args.workload in ("longctx", "kv", "split35", "split25"):
        out["operands"] = OPERANDS_D128
    if "quality" in wl:
        out["quality"] = wl["quality"]()
    if args.workload == "longctx" and not args.no_cpu_baseline:
        W = W_all["longctx"]
        keys, queries = wl["keep"][1], wl["keep"][2]
        out["cpu_baseline"] = cpu_baseline(keys, queries, W["group"], W["bits"], W["seed"],
                                           args.cpu_sample_groups)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
