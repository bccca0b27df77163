"""Benchmark of the quantizer's hot path on one MI355X.

One step = encode every key of the long-context decode workload (norm split,
randomized Hadamard rotation, Lloyd-Max indices, QJL signs: one fused launch)
and score every query head against its KV head's codes (query preparation +
the streaming estimator).  Inputs are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--copy-calibration MIB]

Prints one JSON line.  `value` is scores per second over whole steps; the
per-kernel rates, the roofline of the dominant kernel (algorithmic bytes per
launch / mean HIP-event duration on the launch stream) and the fp64 CPU oracle
timed on a bounded sample of the same workload ride along.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-groups", type=int, default=16)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB three times (untimed), so a "
                         "counter run can scale its byte counters by a copy of known size")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_longctx.json")
KERNEL_SOURCE = os.path.join(ROOT, "rotation_online_vector_amd", "csrc", "kernels.hip")


def measured_traffic(kernel_key):
    """HBM bytes per launch of `kernel_key` from the stored counter runs (FETCH_SIZE and
    WRITE_SIZE scaled by a copy of known size), or None when there is no record or the
    kernel source changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernels_sha256") != src:
        return None
    k = rec.get("kernels", {}).get(kernel_key)
    return None if k is None else k.get("hbm_bytes")


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
    n_scores, dt = 0, 0.0
    for g in range(n_groups):
        s, h = divmod(g, n_kv)
        x = keys[s, h].float().cpu().numpy().astype(np.float64)
        y = queries[s, h * group:(h + 1) * group].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        est = otq.score(plan, otq.encode(plan, x), y)
        dt += time.perf_counter() - t0
        n_scores += est.size
    return {"value": n_scores / dt, "unit": "scores/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d of %d (sequence, KV head) groups: %d keys encoded and scored against "
                      "their %d query heads in fp64 (plan solve excluded), %.1f s of CPU time"
                      % (n_groups, n_seq * n_kv, n_groups * n_tok, group, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only; --gpus %d is not supported (the multi-GPU layout "
              "is described in DESIGN.md, not run)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import rotation_online_vector_amd as tq
    import workloads

    W = workloads.LONGCTX
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    keys, queries, _ = workloads.longctx_inputs(dev)
    n_seq, n_kv, n_tok, d, G = W["n_seq"], W["n_kv"], W["n_tok"], W["d"], W["group"]
    n_keys = n_seq * n_kv * n_tok
    n_groups = n_seq * n_kv
    plan = tq.tq_plan_create(d, W["bits"], W["seed"])
    rb = plan.record_bytes
    codes = torch.empty((n_keys, rb), dtype=torch.uint8, device=dev)
    scores = torch.empty((n_seq * n_kv * G, n_tok), dtype=torch.float32, device=dev)
    xk = keys.view(n_keys, d)
    qv = queries.view(n_groups * G, d)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tq.tq_encode(plan, xk, codes)
        if ev is not None:
            ev[1].record(stream)
        tq.tq_score(plan, qv, codes, n=n_tok, nq_per_group=G, n_groups=n_groups, scores=scores)
        if ev is not None:
            ev[2].record(stream)

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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    sc_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_step = wall * 1e3 / args.steps
    n_scores = n_groups * G * n_tok

    # algorithmic bytes per launch
    enc_bytes = n_keys * d * 2 + n_keys * rb                     # bf16 keys in, records out
    sc_bytes = n_keys * rb + n_scores * 4 + n_groups * G * d * 2  # records + logits + queries
    kern = {
        "tq_encode": {"ms": enc_ms, "bytes": enc_bytes, "gbs": enc_bytes / enc_ms / 1e6,
                      "vectors_per_s": n_keys / enc_ms * 1e3},
        "tq_score": {"ms": sc_ms, "bytes": sc_bytes, "gbs": sc_bytes / sc_ms / 1e6,
                     "scores_per_s": n_scores / sc_ms * 1e3},
    }
    dom = max(kern, key=lambda k: kern[k]["ms"])
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(kern[dom]["gbs"], 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kern[dom]["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom), "bytes_per_launch": kern[dom]["bytes"]}
    out = {
        "metric": "quantized-key scores/sec + HBM GB/s (d=128, 3-bit); encode vectors/sec",
        "value": n_scores / (ms_step / 1e3),
        "unit": "scores/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": W["name"], "n_seq": n_seq, "kv_heads": n_kv, "tokens": n_tok,
                   "d": d, "bits": W["bits"], "query_heads_per_seq": n_kv * G, "gqa_group": G,
                   "keys_per_step": n_keys, "scores_per_step": n_scores, "record_bytes": rb},
        "encode_vectors_per_s": kern["tq_encode"]["vectors_per_s"],
        "score_scores_per_s": kern["tq_score"]["scores_per_s"],
        "kernels": {k: {"ms": round(v["ms"], 4), "alg_bytes": v["bytes"], "alg_gbs": round(v["gbs"], 1),
                        "hbm_frac": round(v["gbs"] / HBM_PEAK_GBS, 4)} for k, v in kern.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(keys, queries, G, W["bits"], W["seed"],
                                           args.cpu_sample_groups)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
