"""TurboQuant-style online vector quantization on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI of libtq (include/tq.h): the functions
below carry the ABI's names and only marshal arguments (tensor pointers, sizes,
the current HIP stream) and allocate output tensors with torch.  Every step of
encode, scoring and top-k runs in the library's HIP kernels; there is no
fallback: if the library is missing or no GPU is present, the calls raise.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libtq.so")

TQ_OK, TQ_EINVAL, TQ_ENOMEM, TQ_EDEVICE, TQ_EUNSUPPORTED = 0, -1, -2, -3, -4
TQ_F32, TQ_BF16 = 0, 1


class TqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, _status_string(status), status))


class tq_subplan_desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("D", ctypes.c_int32), ("R", ctypes.c_int32),
                ("k", ctypes.c_int32), ("record_offset", ctypes.c_int32),
                ("record_bytes", ctypes.c_int32)]


class tq_plan_desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_subplans", ctypes.c_int32),
                ("record_bytes", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("sub", tq_subplan_desc * 2)]


EXPORTED = ["tq_status_string", "tq_plan_create", "tq_plan_destroy", "tq_plan_info",
            "tq_plan_create_mse", "tq_plan_create_heads", "tq_encode", "tq_encode_groups",
            "tq_score", "tq_score_noalloc", "tq_score_topk", "tq_topk",
            "tq_dequantize", "tq_attend", "tq_rerank", "tq_calibrate_outliers",
            "tq_encode_scatter", "tq_qjl", "tq_codebook", "tq_rotation_signs", "tq_qjl_matrix"]

_lib = None


def load_library(path=LIB_PATH):
    """Load libtq.so (after torch, so that both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    try:
        import torch  # noqa: F401  (loads the HIP runtime the library binds to)
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError("libtq.so not built at %s: run `python -m rotation_online_vector_amd.build`"
                           % path)
    lib = ctypes.CDLL(path)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64
    lib.tq_status_string.argtypes = [i32]
    lib.tq_status_string.restype = ctypes.c_char_p
    lib.tq_plan_create.argtypes = [i32, i32, u64, vp, i32, ctypes.POINTER(vp)]
    lib.tq_plan_create.restype = i32
    lib.tq_plan_destroy.argtypes = [vp]
    lib.tq_plan_destroy.restype = None
    lib.tq_plan_info.argtypes = [vp, ctypes.POINTER(tq_plan_desc)]
    lib.tq_plan_info.restype = i32
    lib.tq_encode.argtypes = [vp, vp, i32, i64, i64, vp, vp]
    lib.tq_encode.restype = i32
    lib.tq_encode_groups.argtypes = [vp, vp, i32, i64, i64, i64, vp, vp]
    lib.tq_encode_groups.restype = i32
    lib.tq_plan_create_heads.argtypes = [i32, i32, u64, i32, vp, i32, ctypes.POINTER(vp)]
    lib.tq_plan_create_heads.restype = i32
    lib.tq_score.argtypes = [vp, vp, i32, i64, i64, i64, vp, i64, vp, vp]
    lib.tq_score.restype = i32
    lib.tq_score_noalloc.argtypes = [vp, vp, i32, i64, i64, i64, vp, i64, vp, vp]
    lib.tq_score_noalloc.restype = i32
    lib.tq_topk.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.tq_topk.restype = i32
    lib.tq_plan_create_mse.argtypes = [i32, i32, u64, ctypes.POINTER(vp)]
    lib.tq_plan_create_mse.restype = i32
    lib.tq_dequantize.argtypes = [vp, vp, i64, vp, i32, i64, vp]
    lib.tq_attend.argtypes = [vp, vp, i64, i64, i64, ctypes.c_float, vp, vp, i32, i64, vp]
    lib.tq_attend.restype = i32
    lib.tq_rerank.argtypes = [vp, i32, i64, i64, vp, i32, i64, i64, i32, vp, i32, i32, vp, vp, vp]
    lib.tq_rerank.restype = i32
    lib.tq_calibrate_outliers.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp]
    lib.tq_calibrate_outliers.restype = i32
    lib.tq_encode_scatter.argtypes = [vp, vp, i32, i64, i64, vp, i64, vp, vp]
    lib.tq_encode_scatter.restype = i32
    lib.tq_dequantize.restype = i32
    lib.tq_score_topk.argtypes = [vp, vp, i32, i64, i64, i64, vp, i64, i32, vp, vp, vp]
    lib.tq_score_topk.restype = i32
    lib.tq_qjl.argtypes = [vp, i32, vp, i64, vp, vp]
    lib.tq_qjl.restype = i32
    lib.tq_codebook.argtypes = [i32, i32, vp, vp]
    lib.tq_codebook.restype = i32
    lib.tq_rotation_signs.argtypes = [u64, i32, i32, vp]
    lib.tq_rotation_signs.restype = i32
    lib.tq_qjl_matrix.argtypes = [u64, i32, i32, i32, vp]
    lib.tq_qjl_matrix.restype = i32
    _lib = lib
    return lib


def _status_string(status):
    try:
        return load_library().tq_status_string(status).decode()
    except Exception:
        return "status"


def _check(fn, status):
    if status != TQ_OK:
        raise TqError(fn, status)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    if t.dtype == torch.float32:
        return TQ_F32
    raise TypeError("expected a bfloat16 or float32 tensor, got %s" % t.dtype)


def _on_gpu(*tensors):
    """Every tensor must live on one GPU: the library takes device pointers, and a host
    pointer in a kernel would fault the device."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors passed to the library must be on a GPU (got %s)" % t.device)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors on different devices: %s and %s" % (dev, t.device))


def _out(t, dtype, numel, name):
    """A caller-provided output: contiguous, of the right dtype and at least numel elements,
    so that the library never writes past it."""
    if t.dtype != dtype or not t.is_contiguous() or t.numel() < numel:
        raise ValueError("%s must be contiguous %s with at least %d elements" % (name, dtype, numel))


def _codes(t, nbytes, name="codes"):
    """An input of records: contiguous uint8 holding at least nbytes, since the library reads
    the records as bytes from data_ptr on."""
    import torch
    if t.dtype != torch.uint8 or not t.is_contiguous() or t.numel() < nbytes:
        raise ValueError("%s must be contiguous uint8 with at least %d bytes" % (name, nbytes))


def _groups(rows, nq_per_group, n_groups, what="query rows"):
    """nq_per_group (by default rows / n_groups); empty groups stay empty, as in the C ABI."""
    if n_groups < 0 or (nq_per_group is not None and nq_per_group < 0):
        raise ValueError("group sizes must be >= 0")
    if nq_per_group is None:
        nq_per_group = rows // n_groups if n_groups else 0
    if nq_per_group * n_groups != rows:
        raise ValueError("%s != nq_per_group * n_groups" % what)
    return nq_per_group


def _rows(t, d):
    """(n, ld) of a tensor viewed as rows of d elements with unit inner stride."""
    if t.shape[-1] != d or t.stride(-1) != 1:
        raise ValueError("last dimension must be %d with unit stride" % d)
    if t.dim() == 1:
        return 1, d
    if t.dim() == 2:
        return t.shape[0], t.stride(0)
    if not t.is_contiguous():
        raise ValueError("tensors of rank > 2 must be contiguous")
    return t.numel() // d, d


class Plan:
    """A plan handle (owns the library plan; destroyed with the object)."""

    def __init__(self, handle, desc):
        self._h = handle
        self.desc = desc
        self.d = desc["d"]
        self.record_bytes = desc["record_bytes"]

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan destroyed")
        return self._h

    def __del__(self):
        try:
            tq_plan_destroy(self)
        except Exception:
            pass


def tq_plan_create(d, bits, seed, outlier_mask=None, outlier_bits=0):
    lib = load_library()
    h = ctypes.c_void_p()
    mask_buf = None
    if outlier_mask is not None:
        mask_buf = np.ascontiguousarray(np.asarray(outlier_mask).astype(np.uint8))
        if mask_buf.shape != (d,):
            raise ValueError("outlier_mask must have d entries")
    _check("tq_plan_create", lib.tq_plan_create(
        int(d), int(bits), ctypes.c_uint64(int(seed)),
        None if mask_buf is None else mask_buf.ctypes.data_as(ctypes.c_void_p),
        int(outlier_bits), ctypes.byref(h)))
    return _plan_from_handle(lib, h)


def tq_plan_create_heads(d, bits, seed, outlier_masks, outlier_bits):
    """Layer plan over the heads of a key cache: one outlier mask per head ([n_heads, d],
    each selecting the same number of channels), shared codebooks, rotations and QJL
    matrices; group g of the grouped calls uses head g % n_heads."""
    lib = load_library()
    h = ctypes.c_void_p()
    masks = np.ascontiguousarray(np.asarray(outlier_masks).astype(np.uint8))
    if masks.ndim != 2 or masks.shape[1] != d:
        raise ValueError("outlier_masks must be [n_heads, d]")
    _check("tq_plan_create_heads", lib.tq_plan_create_heads(
        int(d), int(bits), ctypes.c_uint64(int(seed)), int(masks.shape[0]),
        masks.ctypes.data_as(ctypes.c_void_p), int(outlier_bits), ctypes.byref(h)))
    return _plan_from_handle(lib, h)


def tq_plan_create_mse(d, bits, seed):
    """TurboQuant-MSE plan: all b bits on the Lloyd-Max codebook, no QJL stage."""
    lib = load_library()
    h = ctypes.c_void_p()
    _check("tq_plan_create_mse", lib.tq_plan_create_mse(
        int(d), int(bits), ctypes.c_uint64(int(seed)), ctypes.byref(h)))
    return _plan_from_handle(lib, h)


def _plan_from_handle(lib, h):
    desc = tq_plan_desc()
    _check("tq_plan_info", lib.tq_plan_info(h, ctypes.byref(desc)))
    info = {"d": desc.d, "n_subplans": desc.n_subplans, "record_bytes": desc.record_bytes,
            "mode": "mse" if desc.mode == 1 else "inner_product", "n_heads": desc.n_heads,
            "sub": [{f: getattr(desc.sub[i], f) for f, _ in tq_subplan_desc._fields_}
                    for i in range(desc.n_subplans)]}
    return Plan(h, info)


def tq_plan_destroy(plan):
    if plan is not None and plan._h is not None:
        load_library().tq_plan_destroy(plan._h)
        plan._h = None


def tq_plan_info(plan):
    return plan.desc


def tq_encode(plan, x, codes=None, stream=None):
    """Encode the rows of x (cuda bf16/f32, last dim d) into codes (uint8 [n, record_bytes])."""
    import torch
    _on_gpu(x, codes)
    n, ld = _rows(x, plan.d)
    if codes is None:
        codes = torch.empty((n, plan.record_bytes), dtype=torch.uint8, device=x.device)
    _out(codes, torch.uint8, n * plan.record_bytes, "codes")
    _check("tq_encode", load_library().tq_encode(
        plan.handle, ctypes.c_void_p(x.data_ptr()), _dtype_code(x), n, ld,
        ctypes.c_void_p(codes.data_ptr()), _stream(stream)))
    return codes


def tq_encode_groups(plan, x, n_groups, codes=None, stream=None):
    """Records of n_groups equal groups of rows of x ([n_groups * n_per_group, d] or
    [n_groups, n_per_group, d]); with a layer plan, group g uses head g % n_heads."""
    import torch
    _on_gpu(x, codes)
    n, ld = _rows(x, plan.d)
    if n_groups <= 0 or n % n_groups:
        raise ValueError("rows must split into n_groups equal groups")
    if codes is None:
        codes = torch.empty((n, plan.record_bytes), dtype=torch.uint8, device=x.device)
    _out(codes, torch.uint8, n * plan.record_bytes, "codes")
    _check("tq_encode_groups", load_library().tq_encode_groups(
        plan.handle, ctypes.c_void_p(x.data_ptr()), _dtype_code(x), n_groups, n // n_groups, ld,
        ctypes.c_void_p(codes.data_ptr()), _stream(stream)))
    return codes


def tq_score(plan, q, codes, n, nq_per_group=None, n_groups=1, scores=None, stream=None):
    """Scores [n_groups*nq_per_group, n] of query rows q against grouped codes."""
    import torch
    _on_gpu(q, codes, scores)
    nq, ld = _rows(q, plan.d)
    nq_per_group = _groups(nq, nq_per_group, n_groups)
    _codes(codes, n_groups * n * plan.record_bytes)
    if scores is None:
        scores = torch.empty((nq, n), dtype=torch.float32, device=q.device)
    _out(scores, torch.float32, nq * n, "scores")
    _check("tq_score", load_library().tq_score(
        plan.handle, ctypes.c_void_p(q.data_ptr()), _dtype_code(q), nq_per_group, n_groups, ld,
        ctypes.c_void_p(codes.data_ptr()), n, ctypes.c_void_p(scores.data_ptr()), _stream(stream)))
    return scores


def tq_score_noalloc(plan, q, codes, n, scores, nq_per_group=None, n_groups=1, stream=None):
    """tq_score through the entry point that allocates nothing (the query workspace is the
    library's fixed per-device array); `scores` must be provided by the caller."""
    import torch
    if scores is None:
        raise ValueError("tq_score_noalloc writes into a caller-provided scores tensor")
    _on_gpu(q, codes, scores)
    nq, ld = _rows(q, plan.d)
    nq_per_group = _groups(nq, nq_per_group, n_groups)
    _codes(codes, n_groups * n * plan.record_bytes)
    _out(scores, torch.float32, nq * n, "scores")
    _check("tq_score_noalloc", load_library().tq_score_noalloc(
        plan.handle, ctypes.c_void_p(q.data_ptr()), _dtype_code(q), nq_per_group, n_groups, ld,
        ctypes.c_void_p(codes.data_ptr()), n, ctypes.c_void_p(scores.data_ptr()), _stream(stream)))
    return scores


def tq_topk(scores, k, ids=None, vals=None, stream=None):
    import torch
    _on_gpu(scores, ids, vals)
    if scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError("scores must be contiguous float32")
    n = scores.shape[-1]
    nq = scores.numel() // n if n else 0
    if ids is None:
        ids = torch.empty((nq, k), dtype=torch.int64, device=scores.device)
    if vals is None:
        vals = torch.empty((nq, k), dtype=torch.float32, device=scores.device)
    _out(ids, torch.int64, nq * k, "ids")
    _out(vals, torch.float32, nq * k, "vals")
    _check("tq_topk", load_library().tq_topk(
        ctypes.c_void_p(scores.data_ptr()), nq, n, int(k), ctypes.c_void_p(ids.data_ptr()),
        ctypes.c_void_p(vals.data_ptr()), _stream(stream)))
    return ids, vals


def tq_score_topk(plan, q, codes, n, k, nq_per_group=None, n_groups=1, ids=None, vals=None,
                  stream=None):
    """Top-k (ids [rows, k] int64, vals [rows, k] float32) of the scores tq_score would give."""
    import torch
    _on_gpu(q, codes, ids, vals)
    nq, ld = _rows(q, plan.d)
    nq_per_group = _groups(nq, nq_per_group, n_groups)
    _codes(codes, n_groups * n * plan.record_bytes)
    if ids is None:
        ids = torch.empty((nq, k), dtype=torch.int64, device=q.device)
    if vals is None:
        vals = torch.empty((nq, k), dtype=torch.float32, device=q.device)
    _out(ids, torch.int64, nq * k, "ids")
    _out(vals, torch.float32, nq * k, "vals")
    _check("tq_score_topk", load_library().tq_score_topk(
        plan.handle, ctypes.c_void_p(q.data_ptr()), _dtype_code(q), nq_per_group, n_groups, ld,
        ctypes.c_void_p(codes.data_ptr()), n, int(k), ctypes.c_void_p(ids.data_ptr()),
        ctypes.c_void_p(vals.data_ptr()), _stream(stream)))
    return ids, vals


def tq_dequantize(plan, codes, n, x=None, dtype=None, stream=None):
    """Reconstructed vectors [n, d] (float32 or bfloat16) from n records."""
    import torch
    _on_gpu(codes, x)
    _codes(codes, n * plan.record_bytes)
    if x is None:
        x = torch.empty((n, plan.d), dtype=dtype or torch.float32, device=codes.device)
    rows, ld = _rows(x, plan.d)
    if rows != n:
        raise ValueError("output rows != n")
    _check("tq_dequantize", load_library().tq_dequantize(
        plan.handle, ctypes.c_void_p(codes.data_ptr()), n, ctypes.c_void_p(x.data_ptr()),
        _dtype_code(x), ld, _stream(stream)))
    return x


def tq_attend(vplan, logits, vcodes, n, scale, nq_per_group=None, n_groups=1, out=None,
              dtype=None, stream=None):
    """softmax(scale * logits) times the dequantized values, per query row: [rows, d]."""
    import torch
    _on_gpu(logits, vcodes, out)
    if logits.dtype != torch.float32 or not logits.is_contiguous() or logits.shape[-1] != n:
        raise ValueError("logits must be contiguous float32 [rows, n]")
    # n = 0 reaches the library, which rejects it (TQ_EINVAL)
    rows = logits.numel() // n if n else (logits.shape[0] if logits.dim() > 1 else 0)
    nq_per_group = _groups(rows, nq_per_group, n_groups, "logit rows")
    _codes(vcodes, n_groups * n * vplan.record_bytes, "vcodes")
    if out is None:
        out = torch.empty((rows, vplan.d), dtype=dtype or torch.float32, device=logits.device)
    r2, ldo = _rows(out, vplan.d)
    if r2 != rows:
        raise ValueError("output rows != logit rows")
    _check("tq_attend", load_library().tq_attend(
        vplan.handle, ctypes.c_void_p(logits.data_ptr()), nq_per_group, n_groups, n,
        ctypes.c_float(float(scale)), ctypes.c_void_p(vcodes.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), _dtype_code(out), ldo, _stream(stream)))
    return out


def tq_rerank(q, x, cand, k, ids=None, vals=None, stream=None):
    """Exact top-k of each query row over its candidate rows of x (cand: int64 [nq, kc])."""
    import torch
    _on_gpu(q, x, cand, ids, vals)
    d = q.shape[-1]
    nq, ldq = _rows(q, d)
    n, ldx = _rows(x, d)
    if cand.dtype != torch.int64 or not cand.is_contiguous() or cand.dim() != 2 or cand.shape[0] != nq:
        raise ValueError("cand must be contiguous int64 [nq, kc]")
    if ids is None:
        ids = torch.empty((nq, k), dtype=torch.int64, device=q.device)
    if vals is None:
        vals = torch.empty((nq, k), dtype=torch.float32, device=q.device)
    _out(ids, torch.int64, nq * k, "ids")
    _out(vals, torch.float32, nq * k, "vals")
    _check("tq_rerank", load_library().tq_rerank(
        ctypes.c_void_p(q.data_ptr()), _dtype_code(q), nq, ldq, ctypes.c_void_p(x.data_ptr()),
        _dtype_code(x), n, ldx, int(d), ctypes.c_void_p(cand.data_ptr()), int(cand.shape[1]),
        int(k), ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(vals.data_ptr()),
        _stream(stream)))
    return ids, vals


def tq_calibrate_outliers(x, n_out, var=None, mask=None, stream=None):
    """Per-channel variance (fp64) of the rows of x and the mask of its n_out channels of
    largest variance (ties to the lower channel): (var float64 [d], mask uint8 [d])."""
    import torch
    _on_gpu(x, var, mask)
    d = x.shape[-1]
    n, ldx = _rows(x, d)
    if var is None:
        var = torch.empty(d, dtype=torch.float64, device=x.device)
    if mask is None:
        mask = torch.empty(d, dtype=torch.uint8, device=x.device)
    _out(var, torch.float64, d, "var")
    _out(mask, torch.uint8, d, "mask")
    _check("tq_calibrate_outliers", load_library().tq_calibrate_outliers(
        ctypes.c_void_p(x.data_ptr()), _dtype_code(x), n, ldx, int(d), int(n_out),
        ctypes.c_void_p(var.data_ptr()), ctypes.c_void_p(mask.data_ptr()), _stream(stream)))
    return var, mask


def tq_encode_scatter(plan, x, cache, index, stream=None):
    """Encode the rows of x and write record i to row index[i] of cache (uint8
    [rows, record_bytes]); rows outside the cache are skipped."""
    import torch
    _on_gpu(x, cache, index)
    n, ld = _rows(x, plan.d)
    if cache.dtype != torch.uint8 or not cache.is_contiguous() or cache.dim() != 2 or \
            cache.shape[1] != plan.record_bytes:
        raise ValueError("cache must be contiguous uint8 [rows, record_bytes]")
    if index.dtype != torch.int64 or not index.is_contiguous() or index.numel() != n:
        raise ValueError("index must be contiguous int64 [n]")
    _check("tq_encode_scatter", load_library().tq_encode_scatter(
        plan.handle, ctypes.c_void_p(x.data_ptr()), _dtype_code(x), n, ld,
        ctypes.c_void_p(cache.data_ptr()), int(cache.shape[0]), ctypes.c_void_p(index.data_ptr()),
        _stream(stream)))
    return cache


def tq_qjl(plan, subplan, r, beta=None, stream=None):
    import torch
    _on_gpu(r, beta)
    D = plan.desc["sub"][subplan]["D"]
    if r.dtype != torch.float32 or not r.is_contiguous() or r.shape[-1] != D:
        raise ValueError("r must be contiguous float32 [n, D]")
    n = r.numel() // D
    if beta is None:
        beta = torch.empty((n, D // 32), dtype=torch.int32, device=r.device)
    _out(beta, torch.int32, n * (D // 32), "beta")
    _check("tq_qjl", load_library().tq_qjl(
        plan.handle, int(subplan), ctypes.c_void_p(r.data_ptr()), n,
        ctypes.c_void_p(beta.data_ptr()), _stream(stream)))
    return beta


def tq_codebook(D, R):
    lv = np.zeros(2 ** R)
    th = np.zeros(2 ** R - 1)
    _check("tq_codebook", load_library().tq_codebook(
        int(D), int(R), lv.ctypes.data_as(ctypes.c_void_p), th.ctypes.data_as(ctypes.c_void_p)))
    return lv, th


def tq_rotation_signs(seed, subset, D):
    out = np.zeros((3, D), dtype=np.int8)
    _check("tq_rotation_signs", load_library().tq_rotation_signs(
        ctypes.c_uint64(int(seed)), int(subset), int(D), out.ctypes.data_as(ctypes.c_void_p)))
    return out


def tq_qjl_matrix(seed, subset, k, D):
    out = np.zeros((k, D), dtype=np.uint16)
    _check("tq_qjl_matrix", load_library().tq_qjl_matrix(
        ctypes.c_uint64(int(seed)), int(subset), int(k), int(D), out.ctypes.data_as(ctypes.c_void_p)))
    return out
