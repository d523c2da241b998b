"""Plain fp64 CPU oracle of the routed sparse attention layer (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``rt_oracle.c`` (plain C,
float64, sequential loops; see that file's header for the steps and their
page citations) with ctypes.  Inputs are float64 arrays holding the exact
values the device receives; nothing here reads a device result.

Every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, library routines for the special cases the method reduces to, brute
force on tiny inputs, and hand-derived golden values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rt_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile rt_oracle.c with the host C compiler (no HIP anywhere)."""
    stale = (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def route(qk, mu, w: int, nthreads: int | None = None, want_scores: bool = False):
    """O1-O3.  qk [B,H,n,d], mu [H,k,d] -> (inv_norm [B,H,n], idx [B,H,k,w],
    margin [B,H,k], scores [B,H,k,n] or None)."""
    lib = _load()
    qk, mu = _f64(qk), _f64(mu)
    B, H, n, d = qk.shape
    k = mu.shape[1]
    assert mu.shape == (H, k, d) and 1 <= w <= n
    inv = np.empty((B, H, n))
    idx = np.empty((B, H, k, w), dtype=np.int32)
    margin = np.empty((B, H, k))
    scores = np.empty((B, H, k, n)) if want_scores else None
    lib.orc_route_all(_p(qk), _p(mu), ctypes.c_int(B), ctypes.c_int(H), ctypes.c_long(n),
                      ctypes.c_int(d), ctypes.c_int(k), ctypes.c_long(w), _p(inv), _p(idx),
                      _p(margin), _p(scores), ctypes.c_int(nthreads or default_threads()))
    return inv, idx, margin, scores


def routed_attn(q, kk, v, idx, scale: float, causal: bool = True, normalize: bool = True,
                nthreads: int | None = None, want_clusters: bool = False):
    """O1 (if normalize), O4, O5.  -> (out [B,H,n,d], lse [B,H,k,w],
    o_clusters [B,H,k,w,d] or None)."""
    lib = _load()
    q, kk, v, idx = _f64(q), _f64(kk), _f64(v), _i32(idx)
    B, H, n, d = q.shape
    k, w = idx.shape[2], idx.shape[3]
    assert kk.shape == q.shape and v.shape == q.shape and idx.shape[:2] == (B, H)
    assert idx.min() >= 0 and idx.max() < n
    out = np.empty((B, H, n, d))
    lse = np.empty((B, H, k, w))
    oc = np.empty((B, H, k, w, d)) if want_clusters else None
    lib.orc_routed_attn_all(_p(q), _p(kk), _p(v), _p(idx), ctypes.c_int(B), ctypes.c_int(H),
                            ctypes.c_long(n), ctypes.c_int(d), ctypes.c_int(k), ctypes.c_long(w),
                            ctypes.c_double(scale), ctypes.c_int(int(causal)),
                            ctypes.c_int(int(normalize)), _p(out), _p(lse), _p(oc),
                            ctypes.c_int(nthreads or default_threads()))
    return out, lse, oc


def centroid_update(mu, q, kk, idx, lam: float):
    """O1 + O6: returns the updated centroids (the input is not modified)."""
    lib = _load()
    mu2 = _f64(mu).copy()
    q, kk, idx = _f64(q), _f64(kk), _i32(idx)
    B, H, n, d = q.shape
    k, w = idx.shape[2], idx.shape[3]
    assert mu2.shape == (H, k, d)
    lib.orc_centroid_update_all(_p(mu2), _p(q), _p(kk), _p(idx), ctypes.c_int(B), ctypes.c_int(H),
                                ctypes.c_long(n), ctypes.c_int(d), ctypes.c_int(k),
                                ctypes.c_long(w), ctypes.c_double(lam))
    return mu2


def local_attn(q, kk, v, window: int, scale: float, causal: bool = True,
               nthreads: int | None = None):
    """O7 for [B,H,n,d] tensors."""
    lib = _load()
    q, kk, v = _f64(q), _f64(kk), _f64(v)
    B, H, n, d = q.shape
    out = np.empty_like(q)
    lib.orc_local_attn_all(_p(q), _p(kk), _p(v), ctypes.c_int(B), ctypes.c_int(H),
                           ctypes.c_long(n), ctypes.c_int(d), ctypes.c_long(window),
                           ctypes.c_double(scale), ctypes.c_int(int(causal)), _p(out),
                           ctypes.c_int(nthreads or default_threads()))
    return out


def routed_attn_bwd(q, kk, v, idx, dout, scale: float, causal: bool = True,
                    nthreads: int | None = None):
    """O1 + O8: gradients w.r.t. the normalised q^, k^ and v."""
    lib = _load()
    q, kk, v, dout, idx = _f64(q), _f64(kk), _f64(v), _f64(dout), _i32(idx)
    B, H, n, d = q.shape
    k, w = idx.shape[2], idx.shape[3]
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    lib.orc_routed_attn_bwd_all(_p(q), _p(kk), _p(v), _p(idx), _p(dout), ctypes.c_int(B),
                                ctypes.c_int(H), ctypes.c_long(n), ctypes.c_int(d),
                                ctypes.c_int(k), ctypes.c_long(w), ctypes.c_double(scale),
                                ctypes.c_int(int(causal)), _p(dq), _p(dk), _p(dv),
                                ctypes.c_int(nthreads or default_threads()))
    return dq, dk, dv


def local_attn_bwd(q, kk, v, dout, window: int, scale: float, causal: bool = True,
                   nthreads: int | None = None):
    """O9: gradients of O7 w.r.t. q, k and v for [B,H,n,d] tensors."""
    lib = _load()
    q, kk, v, dout = _f64(q), _f64(kk), _f64(v), _f64(dout)
    B, H, n, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    lib.orc_local_attn_bwd_all(_p(q), _p(kk), _p(v), _p(dout), ctypes.c_int(B), ctypes.c_int(H),
                               ctypes.c_long(n), ctypes.c_int(d), ctypes.c_long(window),
                               ctypes.c_double(scale), ctypes.c_int(int(causal)), _p(dq), _p(dk),
                               _p(dv), ctypes.c_int(nthreads or default_threads()))
    return dq, dk, dv


def local_attn_blocked(q, kk, v, block: int, lookback: int, scale: float,
                       nthreads: int | None = None):
    """O10 for [B,H,n,d] tensors (causal blocked local attention)."""
    lib = _load()
    q, kk, v = _f64(q), _f64(kk), _f64(v)
    B, H, n, d = q.shape
    out = np.empty_like(q)
    lib.orc_local_blocked_all(_p(q), _p(kk), _p(v), ctypes.c_int(B), ctypes.c_int(H),
                              ctypes.c_long(n), ctypes.c_int(d), ctypes.c_long(block),
                              ctypes.c_long(lookback), ctypes.c_double(scale), _p(out),
                              ctypes.c_int(nthreads or default_threads()))
    return out


def argmax_labels(x, mu):
    """O1 + O2 + O11: x [B,H,n,d], mu [H,k,d] -> (label [B,H,n] int32, margin
    [B,H,n]: the gap between the largest and the second largest score)."""
    lib = _load()
    x, mu = _f64(x), _f64(mu)
    B, H, n, d = x.shape
    k = mu.shape[1]
    label = np.empty((B, H, n), dtype=np.int32)
    margin = np.empty((B, H, n))
    lib.orc_argmax_all(_p(x), _p(mu), ctypes.c_int(B), ctypes.c_int(H), ctypes.c_long(n),
                       ctypes.c_int(d), ctypes.c_int(k), _p(label), _p(margin))
    return label, margin


def centroid_update_argmax(mu, q, kk, lam: float):
    """O1 + O11: the EMA step with nearest-centroid assignments (the input is
    not modified)."""
    lib = _load()
    mu2 = _f64(mu).copy()
    q, kk = _f64(q), _f64(kk)
    B, H, n, d = q.shape
    k = mu2.shape[1]
    lib.orc_centroid_update_argmax_all(_p(mu2), _p(q), _p(kk), ctypes.c_int(B), ctypes.c_int(H),
                                       ctypes.c_long(n), ctypes.c_int(d), ctypes.c_int(k),
                                       ctypes.c_double(lam))
    return mu2


def route_partition(x, mu):
    """O1 + O2 + O12: partition-style balanced clusters, idx [B,H,k,n/k]."""
    lib = _load()
    x, mu = _f64(x), _f64(mu)
    B, H, n, d = x.shape
    k = mu.shape[1]
    assert n % k == 0
    idx = np.empty((B, H, k, n // k), dtype=np.int32)
    lib.orc_route_partition_all(_p(x), _p(mu), ctypes.c_int(B), ctypes.c_int(H),
                                ctypes.c_long(n), ctypes.c_int(d), ctypes.c_int(k), _p(idx))
    return idx


def normalize_bwd(x, g):
    """Gradient of O1 along the last axis: for x^ = x / r with r = max(||x||,
    1e-12) and the upstream gradient g of x^, dx = (g - x^ <x^, g>) / r while
    ||x|| >= 1e-12 (the Jacobian of x / ||x|| is (I - x^ x^T) / ||x||), and
    dx = g / 1e-12 where the clamp holds r constant."""
    x, g = _f64(x), _f64(g)
    nrm = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    clamped = nrm < 1e-12
    r = np.where(clamped, 1e-12, nrm)
    xhat = x / r
    along = (xhat * g).sum(axis=-1, keepdims=True)
    return np.where(clamped, g / r, (g - xhat * along) / r)


def normalize(x):
    """O1 on the last axis (returns x^ and 1/max(||x||, 1e-12))."""
    lib = _load()
    x = _f64(x)
    d = x.shape[-1]
    n = x.size // d
    xhat = np.empty_like(x)
    inv = np.empty(x.shape[:-1])
    lib.orc_normalize(_p(x), ctypes.c_long(n), ctypes.c_int(d), _p(xhat), _p(inv))
    return xhat, inv


def select(scores, w: int):
    """O3 for scores [k, n] -> (idx [k, w], margin [k])."""
    lib = _load()
    s = _f64(scores)
    k, n = s.shape
    idx = np.empty((k, w), dtype=np.int32)
    margin = np.empty(k)
    lib.orc_select(_p(s), ctypes.c_long(n), ctypes.c_int(k), ctypes.c_long(w), _p(idx), _p(margin))
    return idx, margin


def scores(xhat, mu):
    """O2 for xhat [n, d], mu [k, d] -> s [k, n]."""
    lib = _load()
    xhat, mu = _f64(xhat), _f64(mu)
    n, d = xhat.shape
    k = mu.shape[0]
    s = np.empty((k, n))
    lib.orc_scores(_p(xhat), _p(mu), ctypes.c_long(n), ctypes.c_int(d), ctypes.c_int(k), _p(s))
    return s


def forward(inputs: dict, cfg, scale: float | None = None, nthreads: int | None = None):
    """The whole routed forward of one workload: route, attend, scatter, EMA,
    plus local attention for the local heads.  Returns a dict."""
    qk = inputs["qk"].value
    v = inputs["v"].value
    mu = inputs["mu"]
    sc = (1.0 / np.sqrt(cfg.d)) if scale is None else scale
    inv, idx, margin, _ = route(qk, mu, cfg.w, nthreads)
    out, lse, _ = routed_attn(qk, qk, v, idx, sc, cfg.causal, True, nthreads)
    mu_new = centroid_update(mu, qk, qk, idx, cfg.lam)
    res = {"inv_norm": inv, "idx": idx, "margin": margin, "out": out, "lse": lse,
           "mu": mu_new}
    if cfg.L > 0:
        res["local_out"] = local_attn(inputs["q_local"].value, inputs["k_local"].value,
                                      inputs["v_local"].value, cfg.window, sc, True, nthreads)
    return res


# ---- the layer stack: projections and one layer --------------------------------------
# The paperlayer.ai summary of the paper (§3) describes a self-attention layer as
# three learned linear maps of the n input vectors; §5 reports a 22-layer stack at
# n = 8192.  A stack layer here: [qk | v | q_l | k_l | v_l] = x W_in^T, routed and
# local attention on those heads, y = x + [routed | local] W_o^T.  Activations are
# stored in bfloat16 between the steps, so the oracle rounds at exactly those points
# (the matrix products themselves are exact float64 library products).

def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (8 significant bits), ties to
    even, returned as float64.  Written from the format: x = m 2^e with
    0.5 <= |m| < 1, keep m to 8 bits."""
    f = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(f)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)   # np.round: half to even


def in_proj(x, w_in, R: int, L: int, d: int):
    """x [B,n,dm], w_in [(2R+3L)d, dm] -> (qk, v, q_l, k_l, v_l), each head-major
    [B,H,n,d], rounded to bfloat16 (the local ones None when L = 0)."""
    x, w_in = _f64(x), _f64(w_in)
    B, n, dm = x.shape
    y = round_bf16(x.reshape(B * n, dm) @ w_in.T)            # [B*n, (2R+3L)d]
    heads = y.reshape(B, n, 2 * R + 3 * L, d).transpose(0, 2, 1, 3)
    qk, v = heads[:, :R], heads[:, R:2 * R]
    if L == 0:
        return (np.ascontiguousarray(qk), np.ascontiguousarray(v), None, None, None)
    ql, kl, vl = heads[:, 2 * R:2 * R + L], heads[:, 2 * R + L:2 * R + 2 * L], heads[:, 2 * R + 2 * L:]
    return tuple(np.ascontiguousarray(t) for t in (qk, v, ql, kl, vl))


def out_proj(o_r, o_l, w_o, x=None):
    """y = x + [o_r | o_l] W_o^T, rounded to bfloat16.  o_r [B,R,n,d], o_l
    [B,L,n,d] or None, w_o [dm, (R+L)d], x [B,n,dm] or None."""
    o_r = _f64(o_r)
    B, R, n, d = o_r.shape
    parts = [o_r] if o_l is None else [o_r, _f64(o_l)]
    cat = np.concatenate(parts, axis=1).transpose(0, 2, 1, 3).reshape(B * n, -1)   # [B*n, (R+L)d]
    y = cat @ _f64(w_o).T
    if x is not None:
        y = y + _f64(x).reshape(B * n, -1)
    return round_bf16(y).reshape(B, n, -1)


def layer_forward(x, w_in, w_o, mu, R: int, L: int, d: int, w: int, window: int, lam: float,
                  scale: float | None = None, nthreads: int | None = None):
    """One stack layer (forward, causal, shared query/key in the routed heads).
    Returns a dict with the intermediates: qk, v, q_l, k_l, v_l, idx, margin,
    o_r (routed heads' output, bf16), o_l (local, bf16), mu (updated) and y."""
    sc = (1.0 / np.sqrt(d)) if scale is None else scale
    qk, v, ql, kl, vl = in_proj(x, w_in, R, L, d)
    _, idx, margin, _ = route(qk, mu, w, nthreads)
    o_r, _, _ = routed_attn(qk, qk, v, idx, sc, True, True, nthreads)
    o_r = round_bf16(o_r)
    mu_new = centroid_update(mu, qk, qk, idx, lam)
    o_l = None
    if L > 0:
        o_l = round_bf16(local_attn(ql, kl, vl, window, sc, True, nthreads))
    y = out_proj(o_r, o_l, w_o, x)
    return {"qk": qk, "v": v, "q_l": ql, "k_l": kl, "v_l": vl, "idx": idx, "margin": margin,
            "o_r": o_r, "o_l": o_l, "mu": mu_new, "y": y}


# ---- the layer's backward -------------------------------------------------------------
# Gradients of one stack layer for an upstream gradient dy of y, with the routing
# (the membership) held fixed and the bfloat16 storage roundings of the forward
# taken as the identity.  Where the library stores a value in bfloat16 (the
# gradient of the attention outputs) or feeds a gradient to a bf16 matrix
# product (the gradients of the projected heads), the oracle rounds at the same
# point (rounding=True); rounding=False gives the exact gradient of the exact
# (unrounded) layer, which the finite-difference pins check.

def _heads_to_rows(parts):
    """[B,H_s,n,d] tensors -> [B*n, sum(H_s)*d] (heads concatenated per token)."""
    cat = np.concatenate([_f64(t) for t in parts], axis=1)
    B, H, n, d = cat.shape
    return cat.transpose(0, 2, 1, 3).reshape(B * n, H * d)


def _rows_to_heads(y, B, n, hs, d):
    """[B*n, sum(hs)*d] -> list of [B,h,n,d] tensors."""
    heads = y.reshape(B, n, sum(hs), d).transpose(0, 2, 1, 3)
    out, h0 = [], 0
    for h in hs:
        out.append(np.ascontiguousarray(heads[:, h0:h0 + h]))
        h0 += h
    return out


def out_proj_bwd(dy, o_r, o_l, w_o, rounding: bool = True):
    """Gradients of y = x + [o_r | o_l] W_o^T: returns (do_r, do_l, dw_o); the
    gradient w.r.t. x is dy itself.  do = dy W_o (rounded to bfloat16 when the
    library stores it so), dw_o = dy^T [o_r | o_l]."""
    dy = _f64(dy)
    B, n, dm = dy.shape
    parts = [o_r] if o_l is None else [o_r, o_l]
    hs = [p.shape[1] for p in parts]
    d = o_r.shape[3]
    rows = dy.reshape(B * n, dm)
    do = rows @ _f64(w_o)
    if rounding:
        do = round_bf16(do)
    dw_o = rows.T @ _heads_to_rows(parts)
    outs = _rows_to_heads(do, B, n, hs, d)
    return outs[0], (outs[1] if o_l is not None else None), dw_o


def in_proj_bwd(x, w_in, dqk, dv, dq_l, dk_l, dv_l, dy=None, rounding: bool = True):
    """Gradients of [qk | v | q_l | k_l | v_l] = x W_in^T for the heads'
    gradients (each [B,H_s,n,d]; the local ones None when there are no local
    heads): dx = dC W_in (+ dy, the residual's gradient), dw_in = dC^T x, with
    dC the heads' gradients as token rows (rounded to bfloat16, the products'
    operand precision, when rounding)."""
    x = _f64(x)
    B, n, dm = x.shape
    parts = [dqk, dv] + ([dq_l, dk_l, dv_l] if dq_l is not None else [])
    dc = _heads_to_rows(parts)
    if rounding:
        dc = round_bf16(dc)
    dx = dc @ _f64(w_in)
    if dy is not None:
        dx = dx + _f64(dy).reshape(B * n, dm)
    dw_in = dc.T @ x.reshape(B * n, dm)
    return dx.reshape(B, n, dm), dw_in


def layer_backward(x, w_in, w_o, fwd: dict, dy, R: int, L: int, d: int, window: int,
                   scale: float | None = None, rounding: bool = True,
                   nthreads: int | None = None):
    """Backward of layer_forward (its result dict `fwd`) for the upstream
    gradient dy: out_proj_bwd -> O8 on the routed heads and O9 on the local
    heads -> the normalisation's gradient (q and k share qk, so their two
    gradients add) -> in_proj_bwd.  Returns dx, dw_in, dw_o and the
    intermediate gradients."""
    sc = (1.0 / np.sqrt(d)) if scale is None else scale
    do_r, do_l, dw_o = out_proj_bwd(dy, fwd["o_r"], fwd["o_l"], w_o, rounding)
    qk = fwd["qk"]
    dqh, dkh, dv = routed_attn_bwd(qk, qk, fwd["v"], fwd["idx"], do_r, sc, True, nthreads)
    dqk = normalize_bwd(qk, dqh + dkh)
    dq_l = dk_l = dv_l = None
    if L > 0:
        dq_l, dk_l, dv_l = local_attn_bwd(fwd["q_l"], fwd["k_l"], fwd["v_l"], do_l, window, sc,
                                          True, nthreads)
    dx, dw_in = in_proj_bwd(x, w_in, dqk, dv, dq_l, dk_l, dv_l, dy, rounding)
    return {"do_r": do_r, "do_l": do_l, "dw_o": dw_o, "dq_hat": dqh, "dk_hat": dkh, "dv": dv,
            "dqk": dqk, "dq_l": dq_l, "dk_l": dk_l, "dv_l": dv_l, "dx": dx, "dw_in": dw_in}


# ---- separately routed queries and keys ----------------------------------------------------
# Summary §4 routes queries and keys to the same shared centroids.  With distinct
# query and key vectors each side is routed on its own (O1-O3 on q, and on k), and
# cluster c's queries attend to cluster c's keys with no order between them (the
# content-based sparsity of Summary §4 for data without an order; not causal).

def routed_attn_split(q, kk, v, idx_q, idx_k, scale: float):
    """Queries of cluster c (idx_q[b, h, c]) attend to its keys (idx_k[b, h, c]),
    logit scale * <q^, k^>; each query token sums its rows over the clusters
    that hold it.  -> (out [B,H,n,d], lse [B,H,k,w] (natural log of each query
    row's denominator), sum_q, sum_k [B,H,k,d] (sums of the members' unit rows))."""
    q, kk, v = _f64(q), _f64(kk), _f64(v)
    idx_q, idx_k = _i32(idx_q), _i32(idx_k)
    B, H, n, d = q.shape
    k, w = idx_q.shape[2], idx_q.shape[3]
    assert idx_k.shape == idx_q.shape and kk.shape == q.shape and v.shape == q.shape
    qh, _ = normalize(q)
    kh, _ = normalize(kk)
    out = np.zeros((B, H, n, d))
    lse = np.empty((B, H, k, w))
    sum_q = np.empty((B, H, k, d))
    sum_k = np.empty((B, H, k, d))
    for b in range(B):
        for h in range(H):
            for c in range(k):
                rq, rk = idx_q[b, h, c], idx_k[b, h, c]
                logits = scale * (qh[b, h, rq] @ kh[b, h, rk].T)       # [w queries, w keys]
                m = logits.max(axis=1, keepdims=True)
                e = np.exp(logits - m)
                z = e.sum(axis=1, keepdims=True)
                lse[b, h, c] = (m + np.log(z))[:, 0]
                np.add.at(out[b, h], rq, (e / z) @ v[b, h, rk])
                sum_q[b, h, c] = qh[b, h, rq].sum(axis=0)
                sum_k[b, h, c] = kh[b, h, rk].sum(axis=0)
    return out, lse, sum_q, sum_k


# ---- Jensen-Shannon divergence between local and routed attention --------------------------
# Summary §6 compares, per query, the attention distribution of a local head with that of a
# routing head by the Jensen-Shannon divergence (natural log, so at most ln 2).  Here, for
# every row of every cluster (a query i and one of the clusters holding it), P is the local
# distribution of i (softmax over its window of scale_l * <q_l,i, k_l,j>) and Q the routed one
# (softmax over the cluster's keys visible to i of scale_r * <q^_i, k^_s>); both are written
# out as dense distributions over the n positions.

def attn_js(qk, idx, q_l, k_l, window: int, scale_r: float, scale_l: float, causal: bool = True):
    """-> js [B,H,k,w]: JS(P_local(i) || Q_routed(c, i)) for i = idx[b, h, c, r]."""
    qk, q_l, k_l, idx = _f64(qk), _f64(q_l), _f64(k_l), _i32(idx)
    B, H, n, d = qk.shape
    k, w = idx.shape[2], idx.shape[3]
    xh, _ = normalize(qk)
    js = np.empty((B, H, k, w))
    pos = np.arange(n)
    for b in range(B):
        for h in range(H):
            for c in range(k):
                members = idx[b, h, c]
                for r in range(w):
                    i = members[r]
                    near = (pos <= i) & (pos > i - window) if causal else np.abs(pos - i) < window
                    ll = np.where(near, scale_l * (k_l[b, h] @ q_l[b, h, i]), -np.inf)
                    p = np.exp(ll - ll.max())
                    p /= p.sum()
                    keys = members[:r + 1] if causal else members
                    lr = np.full(n, -np.inf)
                    lr[keys] = scale_r * (xh[b, h, keys] @ xh[b, h, i])
                    q = np.exp(lr - lr.max())
                    q /= q.sum()
                    m = 0.5 * (p + q)
                    kl_p = np.sum(p[p > 0] * np.log(p[p > 0] / m[p > 0]))
                    kl_q = np.sum(q[q > 0] * np.log(q[q > 0] / m[q > 0]))
                    js[b, h, c, r] = 0.5 * (kl_p + kl_q)
    return js


# ---- incremental decode ------------------------------------------------------------------
# Decode-time routing (a reading: the pages' sampling needs one token at a time,
# and the balanced top-w of a whole sequence is not defined for a single new
# token): the new token joins the one cluster whose centroid is nearest (O11),
# its key and value are appended to that cluster's cache, and its query attends
# to every entry of that cache (all at earlier positions or itself, so the step
# is causal).  Local heads keep the last `window` keys and values.  Plain
# float64 numpy; a cache is a dict of arrays.

def decode_cache_from_prefill(qk, v, idx, cap: int):
    """Cluster caches from a prefill membership: for each (b, h, c) the member
    rows of idx[b, h, c] (ascending positions): raw qk rows, their inverse
    norms, values, positions; `cap` entries of room per cluster."""
    qk, v, idx = _f64(qk), _f64(v), _i32(idx)
    B, H, n, d = qk.shape
    k, w = idx.shape[2], idx.shape[3]
    assert cap >= w
    _, inv = normalize(qk)
    ck = np.zeros((B, H, k, cap, d))
    cinv = np.zeros((B, H, k, cap))
    cv = np.zeros((B, H, k, cap, d))
    cpos = np.full((B, H, k, cap), -1, dtype=np.int32)
    clen = np.full((B, H, k), w, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for c in range(k):
                p = idx[b, h, c]
                ck[b, h, c, :w] = qk[b, h, p]
                cinv[b, h, c, :w] = inv[b, h, p]
                cv[b, h, c, :w] = v[b, h, p]
                cpos[b, h, c, :w] = p
    return {"k": ck, "inv": cinv, "v": cv, "pos": cpos, "len": clen}


def decode_step(cache: dict, qk_t, v_t, t: int, mu, scale: float, label_given=None):
    """One routed decode step for the token at position t (qk_t, v_t [B, H, d]):
    returns (out [B, H, d], label [B, H], the updated cache (a copy)).

    ``label_given`` [B, H] (optional): the cluster each (batch, head) joins,
    in place of its own nearest centroid.  Where two centroids are equally
    near within rounding either is a valid choice; a caller that saw the
    other choice taken passes it here so that the caches stay comparable."""
    qk_t, v_t, mu = _f64(qk_t), _f64(v_t), _f64(mu)
    B, H, d = qk_t.shape
    cache = {name: arr.copy() for name, arr in cache.items()}
    out = np.zeros((B, H, d))
    label = np.zeros((B, H), dtype=np.int32)
    cap = cache["k"].shape[3]
    for b in range(B):
        for h in range(H):
            x = qk_t[b, h]
            inv = 1.0 / max(np.sqrt((x * x).sum()), 1e-12)
            s = mu[h] @ (x * inv)
            c = int(np.argmax(s))                      # first maximum: ties to the lower index
            if label_given is not None:
                c = int(label_given[b, h])
            label[b, h] = c
            j = int(cache["len"][b, h, c])
            assert j < cap, "cluster cache full"
            cache["k"][b, h, c, j] = x
            cache["inv"][b, h, c, j] = inv
            cache["v"][b, h, c, j] = v_t[b, h]
            cache["pos"][b, h, c, j] = t
            cache["len"][b, h, c] = j + 1
            keys = cache["k"][b, h, c, :j + 1] * cache["inv"][b, h, c, :j + 1, None]
            logits = scale * (keys @ (x * inv))
            p = np.exp(logits - logits.max())
            p /= p.sum()
            out[b, h] = p @ cache["v"][b, h, c, :j + 1]
    return out, label, cache


def local_decode_step(ring_k, ring_v, q_t, k_t, v_t, t: int, window: int, scale: float):
    """One local decode step: ring_k, ring_v [B, H, window, d] hold position p
    at slot p % window; the new key and value go to slot t % window, and the
    query attends to positions max(0, t - window + 1) .. t.  Returns (out,
    ring_k, ring_v) (copies)."""
    ring_k, ring_v = _f64(ring_k).copy(), _f64(ring_v).copy()
    q_t, k_t, v_t = _f64(q_t), _f64(k_t), _f64(v_t)
    ring_k[:, :, t % window] = k_t
    ring_v[:, :, t % window] = v_t
    pos = np.arange(max(0, t - window + 1), t + 1)
    keys, vals = ring_k[:, :, pos % window], ring_v[:, :, pos % window]   # [B, H, m, d]
    logits = scale * np.einsum("bhmd,bhd->bhm", keys, q_t)
    p = np.exp(logits - logits.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("bhm,bhmd->bhd", p, vals), ring_k, ring_v
