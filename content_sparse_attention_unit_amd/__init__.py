"""Routed sparse attention (Routing Transformer) on MI355X: Python binding.

A thin ctypes layer over ``lib/librouted_attn.so`` (the C ABI declared in
``include/routed_attn.h``).  Every function here only checks tensor
metadata, allocates outputs/workspace with torch on the tensors' device and
passes raw device pointers plus the current HIP stream; all arithmetic runs in
the library's gfx950 kernels.  There is no fallback: if the library is not
built, or a tensor is not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["route", "route_noalloc", "routed_attn", "local_attn", "centroid_update_", "centroid_update_sums_",
           "routed_attn_bwd", "in_proj", "out_proj", "local_attn_bwd", "normalize_bwd",
           "out_proj_bwd", "in_proj_bwd", "local_attn_blocked", "centroid_update_argmax_",
           "route_partition", "routed_attn_split", "routed_attn_update_", "cluster_attn", "scatter_rows", "attn_js", "decode_cache", "decode_fill", "decode_routed",
           "decode_ring_fill", "decode_local", "workspace_bytes", "library_path",
           "mask_words", "RTError", "RT_OP"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "lib", "librouted_attn.so")
_lib = None

RT_F32, RT_BF16 = 0, 1
RT_OP = {"route": 0, "routed_attn": 1, "local_attn": 2, "centroid_update": 3,
         "routed_attn_bwd": 4, "local_attn_bwd": 5, "centroid_update_argmax": 6,
         "route_partition": 7, "attn_js": 8, "routed_attn_update": 9}
_STATUS = {0: "RT_OK", 1: "RT_EINVAL", 2: "RT_EUNSUPPORTED", 3: "RT_EHIP"}


class RTError(RuntimeError):
    """A non-zero rt_status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                           "(or python content_sparse_attention_unit_amd/build.py)")
    lib = ctypes.CDLL(_LIB_PATH)  # torch (imported above) already holds the HIP runtime
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sig = {
        "rt_route": [P, I, P, I, I, I, I, I, I, P, P, P, P, P, P, Z, P],
        "rt_route_noalloc": [P, I, P, I, I, I, I, I, I, P, P, P, P, P],
        "rt_routed_attn": [P, P, P, I, P, P, P, P, I, I, I, I, I, I, F, I, P, I, P, P, P, P, Z,
                           P],
        "rt_centroid_update_sums": [P, P, P, I, I, I, I, F, P],
        "rt_cluster_attn": [P, P, P, I, P, P, P, P, I, I, I, I, I, I, F, I, P, I, P, P, P, P, Z,
                            P],
        "rt_scatter_rows": [P, I, I, I, I, I, I, I, P, I, P, P, P, F, P, Z, P],
        "rt_local_attn": [P, P, P, I, I, I, I, I, I, F, I, P, I, P],
        "rt_centroid_update": [P, P, P, P, P, I, P, I, I, I, I, I, I, F, P],
        "rt_in_proj": [P, P, I, I, I, I, I, I, P, P, P, P, P, P],
        "rt_out_proj": [P, P, P, P, I, I, I, I, I, I, P, P],
        "rt_routed_attn_bwd": [P, P, P, I, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, P,
                               Z, P],
        "rt_local_attn_bwd": [P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, P, Z, P],
        "rt_normalize_bwd": [P, I, P, P, P, ctypes.c_long, I, P, P],
        "rt_out_proj_bwd": [P, P, P, P, I, I, I, I, I, I, P, P, P, P, Z, P],
        "rt_in_proj_bwd": [P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, Z, P],
        "rt_local_attn_blocked": [P, P, P, I, I, I, I, I, I, I, F, P, I, P],
        "rt_centroid_update_argmax": [P, P, P, I, I, I, I, I, I, F, P, Z, P],
        "rt_route_partition": [P, I, P, I, I, I, I, I, P, P, P, P, Z, P],
        "rt_routed_attn_split": [P, P, P, I, P, P, P, P, P, I, I, I, I, I, I, F, P, I, P, P, P, P,
                                 Z, P],
        "rt_routed_attn_update": [P, P, P, I, P, P, P, P, I, I, I, I, I, I, F, I, P, I, P, P, F,
                                  P, Z, P],
        "rt_attn_js": [P, P, P, P, P, I, I, I, I, I, I, I, F, F, I, P, P, Z, P],
        "rt_decode_fill": [P, P, P, P, I, I, I, I, I, I, I, P, P, P, P, P, P],
        "rt_decode_ring_fill": [P, P, I, I, I, I, I, P, P, P],
        "rt_decode_routed": [P, P, P, I, I, I, I, I, P, P, P, P, P, I, F, P, I, P, P],
        "rt_decode_local": [P, P, P, I, I, I, I, P, P, I, F, P, I, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.rt_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.rt_workspace_bytes.restype = ctypes.c_size_t
    lib.rt_proj_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.rt_proj_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.rt_last_error.argtypes = []
    lib.rt_last_error.restype = ctypes.c_char_p
    lib.rt_status_string.argtypes = [I]
    lib.rt_status_string.restype = ctypes.c_char_p
    lib.rt_version.argtypes = []
    lib.rt_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise RTError(status, _load().rt_last_error().decode())


def _ptr(t):
    """A tensor's device address for a c_void_p argument (ctypes takes the int)."""
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    """The current stream of ``device`` as a raw handle (torch's own accessor
    when it has one: no Stream object per call)."""
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RT_F32
    if t.dtype == torch.bfloat16:
        return RT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _gpu(*ts):
    dev, idx = None, -1
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev, idx = t.device, t.get_device()
        elif t.get_device() != idx:
            raise ValueError("all tensors must be on the same device")
    return dev


def _expect(t, shape, dtype, what):
    """Raise ValueError unless ``t`` (if given) has this shape and dtype: the
    kernels index these buffers by the shape arguments alone."""
    if t is None:
        return
    if t.shape != shape:                   # torch.Size is a tuple
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{what} has dtype {t.dtype}, expected {dtype}")


def _check_routed(q, kk, v, idx, q_inv, k_inv, mask=None, lse=None, dout=None, sums=(None, None),
                  mu=None):
    """Metadata checks shared by the routed-attention calls: q, kk, v [B,H,n,d]
    of one dtype, idx int32 [B,H,k,w], inverse norms float32 [B,H,n], the
    membership bitmask int32 [B,H,n,ceil(k/32)] (it must be the one route()
    wrote for this idx), lse float32 [B,H,k,w], dout like q, member sums
    float32 [B,H,k,d], mu float32 [H,k,d]."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, n, d]")
    B, H, n, d = q.shape
    if idx.dim() != 4 or tuple(idx.shape[:2]) != (B, H):
        raise ValueError(f"idx has shape {tuple(idx.shape)}, expected ({B}, {H}, k, w)")
    if idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    k, w = idx.shape[2], idx.shape[3]
    _expect(kk, q.shape, q.dtype, "kk")
    _expect(v, q.shape, q.dtype, "v")
    _expect(q_inv, (B, H, n), torch.float32, "q_inv")
    _expect(k_inv, (B, H, n), torch.float32, "k_inv")
    _expect(mask, (B, H, n, mask_words(k)), torch.int32, "mask")
    _expect(lse, (B, H, k, w), torch.float32, "lse")
    _expect(dout, q.shape, q.dtype, "dout")
    for i, t in enumerate(sums):
        _expect(t, (B, H, k, d), torch.float32, f"sums[{i}]")
    _expect(mu, (H, k, d), torch.float32, "mu")
    return B, H, n, d, k, w


def workspace_bytes(op: str, B: int, H: int, n: int, d: int, k: int, w: int) -> int:
    return int(_load().rt_workspace_bytes(RT_OP[op], B, H, n, d, k, w))


def _workspace(op, dev, B, H, n, d, k, w, ws=None):
    """``ws`` if given (the library checks its size against the call), else a
    new one of rt_workspace_bytes bytes; returns (ws, bytes needed or None)."""
    if ws is not None:
        return ws, None
    need = workspace_bytes(op, B, H, n, d, k, w)
    if need == 0:
        return None, 0
    return torch.empty(need, dtype=torch.uint8, device=dev), need


def mask_words(k: int) -> int:
    return (k + 31) // 32


def route(qk: torch.Tensor, mu: torch.Tensor, w: int, *, want_scores: bool = False,
          want_qk_hat: bool = False, want_mask: bool = False, out=None, ws=None):
    """Normalise, score and select: returns ``(inv_norm, idx)`` plus the
    membership bitmask, ``scores`` and ``qk_hat`` when asked (in that order).
    qk [B,H,n,d] f32/bf16, mu [H,k,d] f32.  ``out`` may carry
    ``(inv_norm, idx)`` or ``(inv_norm, idx, mask)`` preallocated."""
    lib = _load()
    dev = _gpu(qk, mu)
    B, H, n, d = qk.shape
    k = mu.shape[1]
    if mu.dtype != torch.float32 or tuple(mu.shape) != (H, k, d):
        raise ValueError("mu must be float32 [H, k, d]")
    mask = None
    if out is None:
        inv = torch.empty((B, H, n), dtype=torch.float32, device=dev)
        idx = torch.empty((B, H, k, w), dtype=torch.int32, device=dev)
    elif len(out) == 3:
        inv, idx, mask = out
    else:
        inv, idx = out
    if want_mask and mask is None:
        mask = torch.empty((B, H, n, mask_words(k)), dtype=torch.int32, device=dev)
    scores = torch.empty((B, H, k, n), dtype=torch.float32, device=dev) if want_scores else None
    qk_hat = torch.empty_like(qk) if want_qk_hat else None
    if scores is None:
        ws, need = _workspace("route", dev, B, H, n, d, k, w, ws)
    else:
        need = 0
    _check(lib.rt_route(_ptr(qk), _dtype_code(qk), _ptr(mu), B, H, n, d, k, w, _ptr(inv),
                        _ptr(idx), _ptr(mask), _ptr(qk_hat), _ptr(scores), _ptr(ws),
                        0 if ws is None else ws.numel(), _stream(dev)))
    res = [inv, idx]
    if want_mask or (out is not None and len(out) == 3):
        res.append(mask)
    if want_scores:
        res.append(scores)
    if want_qk_hat:
        res.append(qk_hat)
    return tuple(res)


ROUTE_NOALLOC_MAX_SCORES = 16 * 1024 * 1024


def route_noalloc(qk: torch.Tensor, mu: torch.Tensor, w: int, out, *, qk_hat=None):
    """route() through rt_route_noalloc: no workspace, the scores live in the
    library's static per-GPU array (B*H*k*n <= ROUTE_NOALLOC_MAX_SCORES).
    ``out`` = (inv_norm, idx) or (inv_norm, idx, mask), preallocated by the
    caller (this function allocates nothing); returns ``out``."""
    lib = _load()
    inv, idx = out[0], out[1]
    mask = out[2] if len(out) > 2 else None
    dev = _gpu(qk, mu, inv, idx, mask, qk_hat)
    B, H, n, d = qk.shape
    k = mu.shape[1]
    _expect(mu, (H, k, d), torch.float32, "mu")
    _expect(inv, (B, H, n), torch.float32, "inv_norm")
    _expect(idx, (B, H, k, w), torch.int32, "idx")
    _expect(mask, (B, H, n, mask_words(k)), torch.int32, "mask")
    _expect(qk_hat, qk.shape, qk.dtype, "qk_hat")
    _check(lib.rt_route_noalloc(_ptr(qk), _dtype_code(qk), _ptr(mu), B, H, n, d, k, w, _ptr(inv),
                                _ptr(idx), _ptr(mask), _ptr(qk_hat), _stream(dev)))
    return out


def routed_attn(q: torch.Tensor, kk: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                q_inv: torch.Tensor | None = None, k_inv: torch.Tensor | None = None, *,
                scale: float | None = None, causal: bool = True, want_lse: bool = False,
                out_dtype: torch.dtype | None = None, mask: torch.Tensor | None = None,
                sums: tuple | None = None, out=None, lse=None, ws=None):
    """In-cluster attention scatter-added to token order; returns ``out`` (and
    ``lse`` when asked).  Pass ``kk is q`` (and ``k_inv is q_inv``) for shared QK.
    ``out_dtype`` (float32 or bfloat16) defaults to the input dtype; ``mask``
    is the membership bitmask from route(); ``sums`` = (sum_q, sum_k) float32
    [B,H,k,d] tensors (either may be None) to receive per-cluster member sums."""
    lib = _load()
    sum_q, sum_k = sums if sums is not None else (None, None)
    dev = _gpu(q, kk, v, idx, q_inv, k_inv, mask, sum_q, sum_k, out, lse)
    B, H, n, d, k, w = _check_routed(q, kk, v, idx, q_inv, k_inv, mask=mask, lse=lse,
                                     sums=(sum_q, sum_k))
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    _shape(out, q.shape, "out")
    if want_lse and lse is None:
        lse = torch.empty((B, H, k, w), dtype=torch.float32, device=dev)
    ws, _ = _workspace("routed_attn", dev, B, H, n, d, k, w, ws)
    _check(lib.rt_routed_attn(_ptr(q), _ptr(kk), _ptr(v), _dtype_code(q), _ptr(q_inv),
                              _ptr(k_inv), _ptr(idx), _ptr(mask), B, H, n, d, k, w, sc,
                              int(causal), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(sum_q),
                              _ptr(sum_k), _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(dev)))
    return (out, lse) if want_lse else out


def cluster_attn(q, kk, v, idx, q_inv, k_inv, mask, *, scale=None, causal=True, out=None,
                 out_dtype=None, lse=None, sums=(None, None), ws=None):
    """The first stage of routed_attn: in-cluster attention, rows of tokens one
    cluster holds written to ``out``, the others kept in ``ws`` for
    scatter_rows (pass the same ``ws`` and ``out`` there).  ``mask`` (the bits
    route() wrote for idx) is required.  Returns (out, ws)."""
    lib = _load()
    sum_q, sum_k = sums
    dev = _gpu(q, kk, v, idx, q_inv, k_inv, mask, sum_q, sum_k, out, lse)
    if mask is None:
        raise ValueError("cluster_attn needs the membership bits route() wrote")
    B, H, n, d, k, w = _check_routed(q, kk, v, idx, q_inv, k_inv, mask=mask, lse=lse,
                                     sums=(sum_q, sum_k))
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    _shape(out, q.shape, "out")
    ws, _ = _workspace("routed_attn", dev, B, H, n, d, k, w, ws)
    _check(lib.rt_cluster_attn(_ptr(q), _ptr(kk), _ptr(v), _dtype_code(q), _ptr(q_inv),
                               _ptr(k_inv), _ptr(idx), _ptr(mask), B, H, n, d, k, w, sc,
                               int(causal), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(sum_q),
                               _ptr(sum_k), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(dev)))
    return out, ws


def scatter_rows(mask, out, ws, k: int, w: int, *, in_dtype=torch.bfloat16, mu=None,
                 sum_q=None, sum_k=None, lam: float = 0.0):
    """The second stage of routed_attn: sums the rows of tokens several
    clusters hold into ``out`` (ascending centroid order) and zeroes tokens no
    cluster holds; with ``mu`` also the centroid update from sum_q (sum_k).
    ``mask``, ``out``, ``ws`` as given to cluster_attn; ``in_dtype`` is the
    dtype of the attention's inputs.  Returns out."""
    lib = _load()
    dev = _gpu(mask, out, ws, mu, sum_q, sum_k)
    B, H, n, d = out.shape
    _expect(mask, (B, H, n, mask_words(k)), torch.int32, "mask")
    _expect(mu, (H, k, d), torch.float32, "mu")
    _expect(sum_q, (B, H, k, d), torch.float32, "sum_q")
    _expect(sum_k, (B, H, k, d), torch.float32, "sum_k")
    dt = RT_F32 if in_dtype == torch.float32 else RT_BF16
    _check(lib.rt_scatter_rows(_ptr(mask), dt, B, H, n, d, k, w, _ptr(out), _dtype_code(out),
                               _ptr(mu), _ptr(sum_q), _ptr(sum_k), float(lam), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(dev)))
    return out


def local_attn(q: torch.Tensor, kk: torch.Tensor, v: torch.Tensor, window: int, *,
               scale: float | None = None, causal: bool = True,
               out_dtype: torch.dtype | None = None, out=None):
    """Sliding-window attention over [B,H,n,d] tensors; ``out_dtype`` (float32 or
    bfloat16) defaults to the input dtype."""
    lib = _load()
    dev = _gpu(q, kk, v)
    B, H, n, d = q.shape
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    _check(lib.rt_local_attn(_ptr(q), _ptr(kk), _ptr(v), _dtype_code(q), B, H, n, d, int(window),
                             sc, int(causal), _ptr(out), _dtype_code(out), _stream(dev)))
    return out


def centroid_update_(mu: torch.Tensor, q: torch.Tensor, q_inv: torch.Tensor, idx: torch.Tensor,
                     lam: float, kk: torch.Tensor | None = None,
                     k_inv: torch.Tensor | None = None):
    """EMA step of the centroids, in place on ``mu`` [H,k,d] float32."""
    lib = _load()
    dev = _gpu(mu, q, q_inv, idx, kk, k_inv)
    B, H, n, d = q.shape
    k, w = idx.shape[2], idx.shape[3]
    _check(lib.rt_centroid_update(_ptr(mu), _ptr(q), _ptr(q_inv), _ptr(kk), _ptr(k_inv),
                                  _dtype_code(q), _ptr(idx), B, H, n, d, k, w, float(lam),
                                  _stream(dev)))
    return mu


def centroid_update_sums_(mu: torch.Tensor, sum_q: torch.Tensor, lam: float,
                          sum_k: torch.Tensor | None = None):
    """EMA step of the centroids from per-cluster member sums [B,H,k,d]."""
    lib = _load()
    dev = _gpu(mu, sum_q, sum_k)
    B, H, k, d = sum_q.shape
    _check(lib.rt_centroid_update_sums(_ptr(mu), _ptr(sum_q), _ptr(sum_k), B, H, k, d, float(lam),
                                       _stream(dev)))
    return mu


def routed_attn_bwd(q, kk, v, idx, lse, dout, q_inv=None, k_inv=None, *, scale=None,
                    causal=True, mask=None, out=None, ws=None, sum_qk=False):
    """Gradients (dq_hat, dk_hat, dv), float32, of routed_attn for a fixed
    membership; ``lse`` comes from the forward call (want_lse=True), ``mask``
    may be the membership bitmask route() wrote for ``idx`` and ``out`` may
    hold three preallocated float32 [B,H,n,d] tensors.  ``sum_qk`` (shared
    q/k only) returns (dq_hat + dk_hat, None, dv): the gradient of the shared
    normalised vector, with one gradient fewer to scatter; ``out`` may then
    hold (dqk, None, dv)."""
    lib = _load()
    dev = _gpu(q, kk, v, idx, lse, dout, q_inv, k_inv, mask)
    if lse is None or dout is None:
        raise ValueError("routed_attn_bwd needs the forward's lse and dout")
    B, H, n, d, k, w = _check_routed(q, kk, v, idx, q_inv, k_inv, mask=mask, lse=lse, dout=dout)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if sum_qk and (kk is not q or k_inv is not q_inv):
        raise ValueError("sum_qk needs shared q/k (kk is q, k_inv is q_inv)")
    if out is None:
        out = tuple(None if (sum_qk and i == 1) else
                    torch.empty(q.shape, dtype=torch.float32, device=dev) for i in range(3))
    dq, dk, dv = out
    if sum_qk:
        dk = None
    _gpu(dq, dk, dv)
    for name, t in zip(("dq", "dk", "dv"), (dq, dk, dv)):
        if t is None:
            continue
        if t.dtype != torch.float32:
            raise TypeError("gradients are float32")
        _shape(t, q.shape, name)
    ws, _ = _workspace("routed_attn_bwd", dev, B, H, n, d, k, w, ws)
    _check(lib.rt_routed_attn_bwd(_ptr(q), _ptr(kk), _ptr(v), _dtype_code(q), _ptr(q_inv),
                                  _ptr(k_inv), _ptr(idx), _ptr(mask), _ptr(lse), _ptr(dout), B, H,
                                  n, d, k, w,
                                  sc, int(causal), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(dev)))
    return dq, dk, dv


def in_proj(x: torch.Tensor, w_in: torch.Tensor, R: int, L: int, d: int, out=None):
    """[qk | v | q_l | k_l | v_l] = x W_in^T for x [B,n,dm] and w_in
    [(2R+3L)d, dm] (bfloat16); returns the five head-major [B,H,n,d] bfloat16
    tensors (the local ones None when L = 0), or fills ``out``."""
    lib = _load()
    dev = _gpu(x, w_in)
    if x.dtype != torch.bfloat16 or w_in.dtype != torch.bfloat16:
        raise TypeError("in_proj takes bfloat16 tensors")
    B, n, dm = x.shape
    if out is None:
        out = (torch.empty((B, R, n, d), dtype=torch.bfloat16, device=dev),
               torch.empty((B, R, n, d), dtype=torch.bfloat16, device=dev),
               *((torch.empty((B, L, n, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
                 if L > 0 else (None, None, None)))
    _gpu(*out)
    _check(lib.rt_in_proj(_ptr(x), _ptr(w_in), B, n, dm, d, R, L, *(_ptr(t) for t in out),
                          _stream(dev)))
    return out


def out_proj(o_r: torch.Tensor, o_l, w_o: torch.Tensor, x=None, out=None):
    """y = x + [o_r | o_l] W_o^T (bfloat16) for o_r [B,R,n,d], o_l [B,L,n,d] or
    None, w_o [dm, (R+L)d] and the residual x [B,n,dm] or None."""
    lib = _load()
    dev = _gpu(o_r, o_l, w_o, x)
    B, R, n, d = o_r.shape
    L = 0 if o_l is None else o_l.shape[1]
    dm = w_o.shape[0]
    if out is None:
        out = torch.empty((B, n, dm), dtype=torch.bfloat16, device=dev)
    _gpu(out)
    _check(lib.rt_out_proj(_ptr(o_r), _ptr(o_l), _ptr(w_o), _ptr(x), B, n, dm, d, R, L, _ptr(out),
                           _stream(dev)))
    return out


# ---- the layer's backward -------------------------------------------------------------

def local_attn_bwd(q, kk, v, dout, window: int, *, scale=None, causal=True, out=None, ws=None):
    """Gradients (dq, dk, dv), float32, of local_attn (bfloat16 inputs, d in
    {64, 128}); ``out`` may hold three preallocated float32 [B,H,n,d] tensors."""
    lib = _load()
    dev = _gpu(q, kk, v, dout)
    B, H, n, d = q.shape
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = tuple(torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    dq, dk, dv = out
    _gpu(dq, dk, dv)
    ws, _ = _workspace("local_attn_bwd", dev, B, H, n, d, 1, 1, ws)
    _check(lib.rt_local_attn_bwd(_ptr(q), _ptr(kk), _ptr(v), _ptr(dout), _dtype_code(q), B, H, n,
                                 d, int(window), sc, int(causal), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)))
    return dq, dk, dv


def normalize_bwd(x, inv_norm, g1, g2=None, out=None):
    """dx (float32) through x^ = x / max(||x||, 1e-12) for the gradients g1 (+ g2)
    of x^; x [..., d] as given to route, inv_norm from route."""
    lib = _load()
    dev = _gpu(x, inv_norm, g1, g2)
    d = x.shape[-1]
    rows = x.numel() // d
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=dev)
    _gpu(out)
    _check(lib.rt_normalize_bwd(_ptr(x), _dtype_code(x), _ptr(inv_norm), _ptr(g1), _ptr(g2), rows,
                                d, _ptr(out), _stream(dev)))
    return out


def proj_bwd_workspace(B: int, n: int, dm: int, d: int, R: int, L: int, device):
    """A workspace that lets the projections' weight gradients split their
    contraction (None when they would not)."""
    nb = int(_load().rt_proj_bwd_workspace_bytes(B, n, dm, d, R, L))
    return torch.empty(nb, dtype=torch.uint8, device=device) if nb > 0 else None


def _ws_args(ws):
    return (_ptr(ws), 0 if ws is None else ws.numel())


def out_proj_bwd(dy, o_r, o_l, w_o, out=None, ws="auto"):
    """(do_r, do_l, dw_o) for y = x + [o_r | o_l] W_o^T: do_* bfloat16
    head-major (do_l None when there are no local heads), dw_o float32.  ``ws``:
    a workspace for the split weight gradient ("auto": allocated here; None:
    no split)."""
    lib = _load()
    dev = _gpu(dy, o_r, o_l, w_o)
    B, R, n, d = o_r.shape
    L = 0 if o_l is None else o_l.shape[1]
    dm = w_o.shape[0]
    if out is None:
        out = (torch.empty((B, R, n, d), dtype=torch.bfloat16, device=dev),
               torch.empty((B, L, n, d), dtype=torch.bfloat16, device=dev) if L > 0 else None,
               torch.empty((dm, (R + L) * d), dtype=torch.float32, device=dev))
    _gpu(*out)
    if isinstance(ws, str):
        ws = proj_bwd_workspace(B, n, dm, d, R, L, dev)
    _check(lib.rt_out_proj_bwd(_ptr(dy), _ptr(o_r), _ptr(o_l), _ptr(w_o), B, n, dm, d, R, L,
                               *(_ptr(t) for t in out), *_ws_args(ws), _stream(dev)))
    return out


def in_proj_bwd(x, w_in, dqk, dv, dq_l=None, dk_l=None, dv_l=None, dres=None, out=None,
                ws="auto"):
    """(dx, dw_in), float32, for [qk | v | q_l | k_l | v_l] = x W_in^T and the
    heads' float32 gradients; dres (bfloat16 [B,n,dm] or None) is added to dx.
    ``ws`` as in out_proj_bwd."""
    lib = _load()
    dev = _gpu(x, w_in, dqk, dv, dq_l, dk_l, dv_l, dres)
    B, n, dm = x.shape
    R, d = dqk.shape[1], dqk.shape[3]
    L = 0 if dq_l is None else dq_l.shape[1]
    if out is None:
        out = (torch.empty((B, n, dm), dtype=torch.float32, device=dev),
               torch.empty(((2 * R + 3 * L) * d, dm), dtype=torch.float32, device=dev))
    _gpu(*out)
    if isinstance(ws, str):
        ws = proj_bwd_workspace(B, n, dm, d, R, L, dev)
    _check(lib.rt_in_proj_bwd(_ptr(x), _ptr(w_in), _ptr(dqk), _ptr(dv), _ptr(dq_l), _ptr(dk_l),
                              _ptr(dv_l), _ptr(dres), B, n, dm, d, R, L, *(_ptr(t) for t in out),
                              *_ws_args(ws), _stream(dev)))
    return out


# ---- variants ------------------------------------------------------------------------

def local_attn_blocked(q, kk, v, block: int, lookback: int = 1, *, scale=None, out_dtype=None,
                       out=None):
    """Blocked local attention (causal): position i sees its own block of
    `block` positions and the `lookback` blocks before it."""
    lib = _load()
    dev = _gpu(q, kk, v)
    B, H, n, d = q.shape
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    odt = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=dev)
    _gpu(out)
    _check(lib.rt_local_attn_blocked(_ptr(q), _ptr(kk), _ptr(v), _dtype_code(q), B, H, n, d,
                                     int(block), int(lookback), sc, _ptr(out), _dtype_code(out),
                                     _stream(dev)))
    return out


def centroid_update_argmax_(mu, q, kk=None, lam: float = 0.999, ws=None):
    """In-place centroid update with nearest-centroid assignments (each query
    and key counted once, for its own nearest centroid)."""
    lib = _load()
    dev = _gpu(mu, q, kk)
    B, H, n, d = q.shape
    k = mu.shape[1]
    ws, _ = _workspace("centroid_update_argmax", dev, B, H, n, d, k, 1, ws)
    _check(lib.rt_centroid_update_argmax(_ptr(mu), _ptr(q), _ptr(kk), _dtype_code(q), B, H, n, d,
                                         k, float(lam), _ptr(ws),
                                         0 if ws is None else ws.numel(), _stream(dev)))
    return mu


def route_partition(qk, mu, *, want_mask=False, out=None, ws=None):
    """Partition-style balanced routing: returns (inv_norm, idx [B,H,k,n/k])
    and the one-bit-per-token membership mask when asked."""
    lib = _load()
    dev = _gpu(qk, mu)
    B, H, n, d = qk.shape
    k = mu.shape[1]
    if out is None:
        inv = torch.empty((B, H, n), dtype=torch.float32, device=dev)
        idx = torch.empty((B, H, k, n // k), dtype=torch.int32, device=dev)
        mask = (torch.empty((B, H, n, mask_words(k)), dtype=torch.int32, device=dev)
                if want_mask else None)
    else:
        inv, idx, mask = (tuple(out) + (None,))[:3]
    ws, _ = _workspace("route_partition", dev, B, H, n, d, k, 1, ws)
    _check(lib.rt_route_partition(_ptr(qk), _dtype_code(qk), _ptr(mu), B, H, n, d, k, _ptr(inv),
                                  _ptr(idx), _ptr(mask), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(dev)))
    return (inv, idx, mask) if mask is not None else (inv, idx)


def routed_attn_update_(q, kk, v, idx, q_inv, k_inv, mu, lam: float, *, scale=None, causal=True,
                        want_lse=False, out_dtype=None, mask=None, out=None, lse=None, ws=None):
    """routed_attn followed by the centroid update from the same memberships
    (mu updated in place, in the output's scatter launch).  Returns out (and
    lse when asked)."""
    lib = _load()
    dev = _gpu(q, kk, v, idx, q_inv, k_inv, mask, mu, out, lse)
    if mu is None:
        raise ValueError("mu must be float32 [H, k, d]")
    B, H, n, d, k, w = _check_routed(q, kk, v, idx, q_inv, k_inv, mask=mask, lse=lse, mu=mu)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    _shape(out, q.shape, "out")
    if want_lse and lse is None:
        lse = torch.empty((B, H, k, w), dtype=torch.float32, device=dev)
    ws, _ = _workspace("routed_attn_update", dev, B, H, n, d, k, w, ws)
    _check(lib.rt_routed_attn_update(_ptr(q), _ptr(kk), _ptr(v), _dtype_code(q), _ptr(q_inv),
                                     _ptr(k_inv), _ptr(idx), _ptr(mask), B, H, n, d, k, w, sc,
                                     int(causal), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(mu),
                                     float(lam), _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(dev)))
    return (out, lse) if want_lse else out


def routed_attn_split(q, kk, v, idx_q, idx_k, q_inv=None, k_inv=None, *, scale=None,
                      out_dtype=None, q_mask=None, want_lse=False, want_sums=False, out=None,
                      ws=None):
    """Queries and keys routed on their own: cluster c's queries (idx_q) attend
    to its keys and values (idx_k), without a causal mask.  Returns out, plus
    lse and (sum_q, sum_k) when asked."""
    lib = _load()
    dev = _gpu(q, kk, v, idx_q, idx_k, q_inv, k_inv, q_mask)
    B, H, n, d, k, w = _check_routed(q, kk, v, idx_q, q_inv, k_inv, mask=q_mask)
    if tuple(idx_k.shape) != tuple(idx_q.shape):
        raise ValueError("idx_q and idx_k must have the same shape")
    if idx_k.dtype != torch.int32:
        raise TypeError("idx_q and idx_k must be int32")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty((B, H, k, w), dtype=torch.float32, device=dev) if want_lse else None
    sums = (tuple(torch.empty((B, H, k, d), dtype=torch.float32, device=dev) for _ in range(2))
            if want_sums else (None, None))
    ws, _ = _workspace("routed_attn", dev, B, H, n, d, k, w, ws)
    _check(lib.rt_routed_attn_split(_ptr(q), _ptr(kk), _ptr(v), _dtype_code(q), _ptr(q_inv),
                                    _ptr(k_inv), _ptr(idx_q), _ptr(idx_k), _ptr(q_mask), B, H, n,
                                    d, k, w, sc, _ptr(out), _dtype_code(out), _ptr(lse),
                                    _ptr(sums[0]), _ptr(sums[1]), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(dev)))
    res = (out,)
    if want_lse:
        res += (lse,)
    if want_sums:
        res += sums
    return res[0] if len(res) == 1 else res


def attn_js(qk, q_inv, idx, q_l, k_l, window: int, *, scale_r=None, scale_l=None, causal=True,
            out=None, ws=None):
    """Jensen-Shannon divergence [B,H,k,w] between each cluster row's routed
    distribution and its query's local one (a diagnostic; bf16 rows)."""
    lib = _load()
    dev = _gpu(qk, q_inv, idx, q_l, k_l)
    for t_ in (qk, q_l, k_l):
        if t_.dtype != torch.bfloat16:
            raise TypeError("attn_js takes bfloat16 rows")
    B, H, n, d = qk.shape
    k, w = idx.shape[2], idx.shape[3]
    _shape(q_l, qk.shape, "q_l")
    _shape(k_l, qk.shape, "k_l")
    _shape(q_inv, (B, H, n), "q_inv")
    if idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    sr = 1.0 / math.sqrt(d) if scale_r is None else float(scale_r)
    sl = 1.0 / math.sqrt(d) if scale_l is None else float(scale_l)
    if out is None:
        out = torch.empty((B, H, k, w), dtype=torch.float32, device=dev)
    _shape(out, (B, H, k, w), "out")
    ws, _ = _workspace("attn_js", dev, B, H, n, d, k, w, ws)
    _check(lib.rt_attn_js(_ptr(qk), _ptr(q_inv), _ptr(idx), _ptr(q_l), _ptr(k_l), B, H, n, d, k,
                          w, int(window), sr, sl, int(bool(causal)), _ptr(out), _ptr(ws),
                          0 if ws is None else ws.numel(), _stream(dev)))
    return out


# ---- incremental decode ------------------------------------------------------------------

def _bf16(*ts):
    for t in ts:
        if t.dtype != torch.bfloat16:
            raise TypeError("decode takes bfloat16 rows")


def _shape(t, want, what):
    if t.shape != tuple(want):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _check_cache(cache, B, H, k, cap, d):
    _shape(cache["k"], (B, H, k, cap, d), "cache k")
    _shape(cache["v"], (B, H, k, cap, d), "cache v")
    _shape(cache["inv"], (B, H, k, cap), "cache inv")
    _shape(cache["pos"], (B, H, k, cap), "cache pos")
    _shape(cache["len"], (B, H, k), "cache len")
    for name, dt in (("k", torch.bfloat16), ("v", torch.bfloat16), ("inv", torch.float32),
                     ("pos", torch.int32), ("len", torch.int32)):
        if cache[name].dtype != dt:
            raise TypeError(f"cache {name} must be {dt}")


def decode_cache(B: int, H: int, k: int, cap: int, d: int, device) -> dict:
    """Empty cluster caches (positions -1, no entries in use)."""
    return {"k": torch.zeros((B, H, k, cap, d), dtype=torch.bfloat16, device=device),
            "inv": torch.zeros((B, H, k, cap), dtype=torch.float32, device=device),
            "v": torch.zeros((B, H, k, cap, d), dtype=torch.bfloat16, device=device),
            "pos": torch.full((B, H, k, cap), -1, dtype=torch.int32, device=device),
            "len": torch.zeros((B, H, k), dtype=torch.int32, device=device)}


def decode_fill(qk, v, inv, idx, cap: int, cache=None) -> dict:
    """Cluster caches from a prefill membership (idx [B,H,k,w], inv [B,H,n])."""
    lib = _load()
    dev = _gpu(qk, v, inv, idx)
    _bf16(qk, v)
    B, H, n, d = qk.shape
    k, w = idx.shape[2], idx.shape[3]
    _shape(v, qk.shape, "v")
    _shape(inv, (B, H, n), "inv")
    _shape(idx[:, :, 0, 0], (B, H), "idx")
    if idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    if cache is None:
        cache = decode_cache(B, H, k, cap, d, dev)
    _check_cache(cache, B, H, k, cap, d)
    _check(lib.rt_decode_fill(_ptr(qk), _ptr(inv), _ptr(v), _ptr(idx), B, H, n, d, k, w, int(cap),
                              _ptr(cache["k"]), _ptr(cache["inv"]), _ptr(cache["v"]),
                              _ptr(cache["pos"]), _ptr(cache["len"]), _stream(dev)))
    return cache


def decode_routed(cache: dict, qk_t, v_t, t: int, mu, *, scale=None, out_dtype=None, out=None,
                  label=None):
    """One routed decode step (the caches are appended to in place); returns
    (out [B,H,d], label [B,H])."""
    lib = _load()
    dev = _gpu(qk_t, v_t, mu, *cache.values())
    _bf16(qk_t, v_t)
    B, H, d = qk_t.shape
    k, cap = cache["k"].shape[2], cache["k"].shape[3]
    _shape(v_t, (B, H, d), "v_t")
    _shape(mu, (H, k, d), "mu")
    if mu.dtype != torch.float32:
        raise TypeError("mu must be float32")
    _check_cache(cache, B, H, k, cap, d)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype or qk_t.dtype, device=dev)
    _shape(out, (B, H, d), "out")
    if label is None:
        label = torch.empty((B, H), dtype=torch.int32, device=dev)
    _gpu(out, label)
    _shape(label, (B, H), "label")
    _check(lib.rt_decode_routed(_ptr(qk_t), _ptr(v_t), _ptr(mu), B, H, d, k, cap,
                                _ptr(cache["k"]), _ptr(cache["inv"]), _ptr(cache["v"]),
                                _ptr(cache["pos"]), _ptr(cache["len"]), int(t), sc, _ptr(out),
                                _dtype_code(out), _ptr(label), _stream(dev)))
    return out, label


def decode_ring_fill(kk, v, window: int, ring=None):
    """The local rings (ring_k, ring_v [B,H,window,d]) from a prefill's keys and values."""
    lib = _load()
    dev = _gpu(kk, v)
    _bf16(kk, v)
    B, H, n, d = kk.shape
    _shape(v, kk.shape, "v")
    if ring is None:
        ring = (torch.zeros((B, H, window, d), dtype=torch.bfloat16, device=dev),
                torch.zeros((B, H, window, d), dtype=torch.bfloat16, device=dev))
    _bf16(*ring)
    _shape(ring[0], (B, H, window, d), "ring_k")
    _shape(ring[1], (B, H, window, d), "ring_v")
    _check(lib.rt_decode_ring_fill(_ptr(kk), _ptr(v), B, H, n, d, int(window), _ptr(ring[0]),
                                   _ptr(ring[1]), _stream(dev)))
    return ring


def decode_local(ring_k, ring_v, q_t, k_t, v_t, t: int, *, scale=None, out_dtype=None, out=None):
    """One local decode step (the rings are written in place); returns out [B,H,d]."""
    lib = _load()
    dev = _gpu(ring_k, ring_v, q_t, k_t, v_t)
    _bf16(ring_k, ring_v, q_t, k_t, v_t)
    B, H, d = q_t.shape
    window = ring_k.shape[2]
    for t_, what in ((k_t, "k_t"), (v_t, "v_t")):
        _shape(t_, (B, H, d), what)
    _shape(ring_k, (B, H, window, d), "ring_k")
    _shape(ring_v, (B, H, window, d), "ring_v")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype or q_t.dtype, device=dev)
    _gpu(out)
    _shape(out, (B, H, d), "out")
    _check(lib.rt_decode_local(_ptr(q_t), _ptr(k_t), _ptr(v_t), B, H, d, window, _ptr(ring_k),
                               _ptr(ring_v), int(t), sc, _ptr(out), _dtype_code(out),
                               _stream(dev)))
    return out
