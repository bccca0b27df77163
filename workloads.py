"""Seeded synthetic inputs for the five benchmark shapes.

This module draws input data only; it holds none of the quantizer's
arithmetic, and both the HIP path and the CPU oracle consume the exact bytes
it produces.  Small shapes are drawn with numpy on the host; the large
key-cache shapes are drawn with torch on the device that will consume them
(a seeded torch.Generator of that device), and the oracle receives copies of
the sampled rows.

Shapes (all keys/queries are row vectors of the key dimension):
  small   : 4096 keys x 128, 64 queries, fp32 i.i.d. N(0, 1); b = 4
  kv      : 8 KV heads x 32768 tokens x 128, bf16 N(0, 1), 4 channels per head
            (seeded) scaled x10; 32 query heads (GQA group 4); b = 3
  split   : 8 KV heads x 65536 tokens x 128, bf16, 32 channels per head scaled
            x10 and marked as outliers; b = 3 / outlier b = 5 (or 2 / 4)
  retrieval: 1,000,000 x 1536 fp32 unit vectors, anisotropic Gaussian with
            eigenvalues 1/i along the axes; 1024 queries of the same law; b = 4
  longctx : 16 sequences x 8 KV heads x 131072 tokens x 128, bf16 N(0, 1) with
            6 channels per (sequence, head) drawn Student-t (3 d.o.f.); b = 3
  attend  : the longctx keys (b = 3) and values drawn the same way with seed 1
            (3-bit MSE plan), both held encoded; one decode step scores and attends
  decode  : the attend caches; a step appends one token per (sequence, KV head) to both
            caches (at the last slot, so the length stays 131072), then scores and attends
  msekeys : the longctx keys under the 3-bit MSE plan, encoded and scored
  retrievalmse: the retrieval vectors as a 4-bit MSE index, encoded and searched (top-10)
  decodemse: the decode step with the keys also under the 3-bit MSE plan
"""
import numpy as np

SMALL = dict(name="small-d128-N4096-q64-b4", n_keys=4096, n_queries=64, d=128, bits=4, seed=0)
KV = dict(name="kv-8x32768x128-bf16-b3", n_kv=8, n_tok=32768, d=128, group=4, bits=3,
          n_outlier=4, outlier_scale=10.0, seed=0)
SPLIT = dict(name="split-8x65536x128-bf16-b3o5", n_kv=8, n_tok=65536, d=128, group=4,
             bits=3, outlier_bits=5, n_outlier=32, outlier_scale=10.0, seed=0)
SPLIT_25 = dict(SPLIT, name="split-8x65536x128-bf16-b2o4", bits=2, outlier_bits=4)
RETRIEVAL = dict(name="retrieval-1e6x1536-fp32-b4", n_keys=1_000_000, n_queries=1024, d=1536,
                 bits=4, topk=10, seed=0)
LONGCTX = dict(name="longctx-16x8x131072x128-bf16-b3", n_seq=16, n_kv=8, n_tok=131072, d=128,
               group=4, bits=3, n_heavy=6, dof=3, seed=0)
# TurboQuant-MSE on the same keys: 3-bit codes for most heads (technical overview §4.1.1),
# dequantized in one batch before attention (§4.1.2)
MSE_LONGCTX = dict(LONGCTX, name="mse-longctx-16x8x131072x128-bf16-b3")
# the same keys held under the 3-bit MSE plan and scored (overview §4.1.1: 3-bit MSE for most
# heads), and the retrieval shape as an MSE index (§4.2.1: every vector MSE-quantized, its
# norm kept) searched by the quantized distance of §4.2.2
MSEKEYS_LONGCTX = dict(LONGCTX, name="msekeys-longctx-16x8x131072x128-bf16-m3")
RETRIEVAL_MSE = dict(RETRIEVAL, name="retrieval-mse-1e6x1536-fp32-m4")
# one decode step over the same cache held quantized: keys under the inner-product plan
# (scored), values under a 3-bit MSE plan (attended), both encoded before the step
ATTEND_LONGCTX = dict(LONGCTX, name="attend-longctx-16x8x131072x128-k3ip-v3mse",
                      v_bits=3, v_seed=1)
# a whole decode step over that cache: one new token per (sequence, KV head) appended to the
# key and value caches (overview §4.1.2), then scoring and attention over all 131072 tokens
DECODE_LONGCTX = dict(ATTEND_LONGCTX, name="decode-longctx-16x8x131072x128-k3ip-v3mse")
# the decode step with both caches under 3-bit MSE plans (the most-heads case of §4.1.1)
DECODE_MSE_LONGCTX = dict(DECODE_LONGCTX, name="decode-longctx-16x8x131072x128-k3mse-v3mse")


def small_inputs(n_keys=4096, n_queries=64, d=128, seed=0):
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((n_keys, d)).astype(np.float32)
    queries = rng.standard_normal((n_queries, d)).astype(np.float32)
    return keys, queries


def outlier_channels(n_heads, d, n_outlier, seed=0):
    """Per head, a seeded choice of n_outlier distinct channels (sorted)."""
    rng = np.random.default_rng(seed)
    return np.stack([np.sort(rng.choice(d, n_outlier, replace=False)) for _ in range(n_heads)])


def _torch_gen(device, seed):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def kv_inputs(device, n_kv=8, n_tok=32768, d=128, group=4, n_outlier=4, outlier_scale=10.0,
              seed=0, dtype="bfloat16"):
    """Keys [n_kv, n_tok, d] with n_outlier scaled channels per head, queries [n_kv*group, d].

    Returns (keys, queries, channels[n_kv, n_outlier])."""
    import torch
    dt = getattr(torch, dtype)
    g = _torch_gen(device, seed)
    ch = outlier_channels(n_kv, d, n_outlier, seed)
    keys = torch.randn((n_kv, n_tok, d), generator=g, device=device, dtype=torch.float32)
    scale = torch.ones((n_kv, 1, d), device=device)
    for h in range(n_kv):
        scale[h, 0, torch.as_tensor(ch[h], device=device)] = outlier_scale
    keys = (keys * scale).to(dt)
    queries = torch.randn((n_kv * group, d), generator=g, device=device,
                          dtype=torch.float32).to(dt)
    return keys, queries, ch


def retrieval_inputs(device, n_keys=1_000_000, n_queries=1024, d=1536, seed=0, chunk=1 << 17):
    """Unit-norm keys and queries: x = (g * sqrt(lambda)) / ||.||, lambda_i = 1/i, g ~ N(0, I)."""
    import torch
    g = _torch_gen(device, seed)
    sd = torch.rsqrt(torch.arange(1, d + 1, device=device, dtype=torch.float32))

    def draw(n):
        out = torch.empty((n, d), device=device, dtype=torch.float32)
        for s in range(0, n, chunk):
            e = min(n, s + chunk)
            x = torch.randn((e - s, d), generator=g, device=device, dtype=torch.float32) * sd
            out[s:e] = x / torch.linalg.vector_norm(x, dim=1, keepdim=True)
        return out

    keys = draw(n_keys)
    queries = draw(n_queries)
    return keys, queries


def longctx_inputs(device, n_seq=16, n_kv=8, n_tok=131072, d=128, group=4, n_heavy=6, dof=3,
                   seed=0):
    """Keys [n_seq, n_kv, n_tok, d] bf16 N(0, 1) except n_heavy channels per
    (sequence, head) drawn Student-t with `dof` degrees of freedom (unscaled);
    queries [n_seq, n_kv*group, d] bf16 N(0, 1).  Returns (keys, queries, channels)."""
    import torch
    g = _torch_gen(device, seed)
    ch = outlier_channels(n_seq * n_kv, d, n_heavy, seed).reshape(n_seq, n_kv, n_heavy)
    keys = torch.empty((n_seq, n_kv, n_tok, d), device=device, dtype=torch.bfloat16)
    for s in range(n_seq):
        x = torch.randn((n_kv, n_tok, d), generator=g, device=device, dtype=torch.float32)
        z = torch.randn((n_kv, n_tok, n_heavy), generator=g, device=device, dtype=torch.float32)
        chi = torch.randn((n_kv, n_tok, n_heavy, dof), generator=g, device=device,
                          dtype=torch.float32).square().sum(-1)
        t = z / torch.sqrt(chi / dof)
        idx = torch.as_tensor(ch[s], device=device, dtype=torch.int64)      # [n_kv, n_heavy]
        x.scatter_(2, idx[:, None, :].expand(n_kv, n_tok, n_heavy), t)
        keys[s] = x.to(torch.bfloat16)
    queries = torch.randn((n_seq, n_kv * group, d), generator=g, device=device,
                          dtype=torch.float32).to(torch.bfloat16)
    return keys, queries, ch
