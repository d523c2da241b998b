"""CPU tests of the C ABI: the library loads, exports every function declared
in include/routed_attn.h, and rejects invalid arguments on the host before
anything is enqueued (no GPU is touched: each call below fails validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "routed_attn.h")

RT_OK, RT_EINVAL, RT_EUNSUPPORTED = 0, 1, 2
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call fails validation first


@pytest.fixture(scope="module")
def lib():
    import content_sparse_attention_unit_amd as rt
    return rt._load()


def _last(lib):
    return lib.rt_last_error().decode()


def test_exports_every_declared_function(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:rt_status|size_t|const char \*|int)\s*\*?\s*(rt_\w+)\s*\(",
                              text, flags=re.M))
    assert {"rt_route", "rt_routed_attn", "rt_local_attn", "rt_centroid_update",
            "rt_centroid_update_sums", "rt_routed_attn_bwd", "rt_workspace_bytes", "rt_status_string", "rt_last_error",
            "rt_version"} <= declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for code in range(4):
        assert lib.rt_status_string(code).startswith(b"RT_")
    assert lib.rt_version() >= 10000


def route(lib, qk=FAKE, dtype=1, mu=FAKE, B=1, H=1, n=64, d=16, k=4, w=16, inv=FAKE, idx=FAKE,
          scores=None, ws=FAKE, ws_bytes=1 << 30):
    return lib.rt_route(qk, dtype, mu, B, H, n, d, k, w, inv, idx, None, None, scores, ws, ws_bytes,
                        None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(qk=None), RT_EINVAL, "null"),
    (dict(mu=None), RT_EINVAL, "null"),
    (dict(inv=None), RT_EINVAL, "null"),
    (dict(idx=None), RT_EINVAL, "null"),
    (dict(B=0), RT_EINVAL, "positive"),
    (dict(n=-1), RT_EINVAL, "positive"),
    (dict(k=0), RT_EINVAL, "positive"),
    (dict(w=0), RT_EINVAL, "positive"),
    (dict(w=65), RT_EINVAL, "exceeds n"),
    (dict(d=48), RT_EUNSUPPORTED, "d=48"),
    (dict(dtype=7), RT_EUNSUPPORTED, "dtype"),
    (dict(n=70000, w=16), RT_EUNSUPPORTED, "exceeds 65536"),
    (dict(B=300, H=300), RT_EUNSUPPORTED, "B*H"),
    (dict(ws=None), RT_EINVAL, "workspace"),
    (dict(ws_bytes=100), RT_EINVAL, "workspace"),
])
def test_route_validation(lib, kw, code, msg):
    assert route(lib, **kw) == code
    assert msg in _last(lib)


def route_noalloc(lib, qk=FAKE, dtype=1, mu=FAKE, B=1, H=1, n=64, d=16, k=4, w=16, inv=FAKE,
                  idx=FAKE):
    return lib.rt_route_noalloc(qk, dtype, mu, B, H, n, d, k, w, inv, idx, None, None, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(qk=None), RT_EINVAL, "null"),
    (dict(idx=None), RT_EINVAL, "null"),
    (dict(w=65), RT_EINVAL, "exceeds n"),
    (dict(d=48), RT_EUNSUPPORTED, "d=48"),
    (dict(B=1, H=8, n=32768, k=128, w=256), RT_EUNSUPPORTED, "static scratch"),
    (dict(B=2, H=1, n=65536, k=129, w=16), RT_EUNSUPPORTED, "static scratch"),
])
def test_route_noalloc_validation(lib, kw, code, msg):
    """Checked on the host before the scratch array is looked up or anything
    is launched; the limit is RT_ROUTE_NOALLOC_MAX_SCORES scores."""
    assert route_noalloc(lib, **kw) == code
    assert msg in _last(lib)


def route_partition(lib, qk=FAKE, dtype=1, mu=FAKE, B=1, H=1, n=64, d=16, k=4, inv=FAKE,
                    idx=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.rt_route_partition(qk, dtype, mu, B, H, n, d, k, inv, idx, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(qk=None), RT_EINVAL, "null"),
    (dict(idx=None), RT_EINVAL, "null"),
    (dict(k=0), RT_EINVAL, "positive"),
    (dict(k=257, n=257 * 4), RT_EUNSUPPORTED, "k=257"),
    (dict(n=100, k=8), RT_EINVAL, "multiple"),
    (dict(n=32768, k=64), RT_EUNSUPPORTED, "exceeds 16384"),
    (dict(ws=None), RT_EINVAL, "workspace"),
    (dict(ws_bytes=64 * 16 + 5 * 4 - 1), RT_EINVAL, "workspace"),
    (dict(d=48), RT_EUNSUPPORTED, "d=48"),
])
def test_route_partition_validation(lib, kw, code, msg):
    """Checked on the host before anything is launched: n a multiple of k,
    n <= 16384, k <= 256, and the workspace rt_workspace_bytes names."""
    assert route_partition(lib, **kw) == code
    assert msg in _last(lib)


def test_route_partition_workspace(lib):
    # label, best, group list and cluster per token (4 bytes each), then k + 1
    # group offsets per (batch, head)
    B, H, n, d, k = 2, 3, 8192, 128, 64
    assert lib.rt_workspace_bytes(7, B, H, n, d, k, 1) == B * H * n * 16 + B * H * (k + 1) * 4


def test_route_noalloc_limit_matches_header():
    import content_sparse_attention_unit_amd as rt
    text = open(HEADER).read()
    m = re.search(r"#define RT_ROUTE_NOALLOC_MAX_SCORES \((\d+) \* (\d+) \* (\d+)\)", text)
    assert m and int(m[1]) * int(m[2]) * int(m[3]) == rt.ROUTE_NOALLOC_MAX_SCORES


def attn(lib, q=FAKE, kk=FAKE, v=FAKE, dtype=1, q_inv=FAKE, k_inv=FAKE, idx=FAKE, B=1, H=1,
         n=64, d=16, k=4, w=16, scale=0.25, causal=1, out=ctypes.c_void_p(0x2000), out_dtype=1,
         lse=None, ws=FAKE, ws_bytes=0):
    return lib.rt_routed_attn(q, kk, v, dtype, q_inv, k_inv, idx, None, B, H, n, d, k, w, scale,
                              causal, out, out_dtype, lse, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), RT_EINVAL, "null"),
    (dict(v=None), RT_EINVAL, "null"),
    (dict(idx=None), RT_EINVAL, "null"),
    (dict(out=None), RT_EINVAL, "null"),
    (dict(k_inv=None), RT_EINVAL, "both"),
    (dict(w=65), RT_EINVAL, "exceeds n"),
    (dict(k=257), RT_EUNSUPPORTED, "k=257"),
    (dict(d=8), RT_EUNSUPPORTED, "d=8"),
    (dict(out=FAKE), RT_EINVAL, "alias"),
    (dict(scale=float("inf")), RT_EINVAL, "scale"),
    (dict(scale=float("nan")), RT_EINVAL, "scale"),
    (dict(causal=2), RT_EINVAL, "causal"),
    (dict(n=4096, d=128, w=300), RT_EUNSUPPORTED, "w=300"),
    (dict(n=4096, d=64, w=600), RT_EUNSUPPORTED, "w=600"),
    (dict(ws_bytes=10), RT_EINVAL, "workspace"),
    (dict(out_dtype=5), RT_EUNSUPPORTED, "out_dtype"),
])
def test_routed_attn_validation(lib, kw, code, msg):
    assert attn(lib, **kw) == code
    assert msg in _last(lib)


def cluster(lib, mask=FAKE, B=1, H=1, n=64, d=16, k=4, w=16, ws_bytes=1 << 30):
    return lib.rt_cluster_attn(FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, mask, B, H, n, d, k, w, 0.25,
                               1, ctypes.c_void_p(0x2000), 1, None, None, None, FAKE, ws_bytes,
                               None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(mask=None), RT_EINVAL, "member_mask"),
    (dict(w=65), RT_EINVAL, "exceeds n"),
    (dict(d=48), RT_EUNSUPPORTED, "d=48"),
    (dict(ws_bytes=10), RT_EINVAL, "workspace"),
])
def test_cluster_attn_validation(lib, kw, code, msg):
    assert cluster(lib, **kw) == code
    assert msg in _last(lib)


def scatter(lib, mask=FAKE, dtype=1, B=1, H=1, n=64, d=16, k=4, w=16, out=FAKE, out_dtype=1,
            mu=None, sum_q=None, lam=0.5, ws=FAKE, ws_bytes=1 << 30):
    return lib.rt_scatter_rows(mask, dtype, B, H, n, d, k, w, out, out_dtype, mu, sum_q, None,
                               lam, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(mask=None), RT_EINVAL, "null"),
    (dict(out=None), RT_EINVAL, "null"),
    (dict(mu=FAKE), RT_EINVAL, "sum_q"),
    (dict(mu=FAKE, sum_q=FAKE, lam=1.5), RT_EINVAL, "lambda"),
    (dict(n=0), RT_EINVAL, "positive"),
    (dict(k=300), RT_EUNSUPPORTED, "k=300"),
    (dict(d=8), RT_EUNSUPPORTED, "d=8"),
    (dict(dtype=3), RT_EUNSUPPORTED, "dtype"),
    (dict(out_dtype=4), RT_EUNSUPPORTED, "out_dtype"),
    (dict(ws=None), RT_EINVAL, "workspace"),
    (dict(ws_bytes=100), RT_EINVAL, "workspace"),
])
def test_scatter_rows_validation(lib, kw, code, msg):
    assert scatter(lib, **kw) == code
    assert msg in _last(lib)


def test_routed_attn_limits_depend_on_sharing(lib):
    # distinct q/k at d=128 is limited to w=128, shared q/k to 256
    assert attn(lib, q=ctypes.c_void_p(0x3000), n=4096, d=128, w=200, ws_bytes=0) == RT_EUNSUPPORTED
    assert attn(lib, q=FAKE, kk=FAKE, n=4096, d=128, w=200, ws_bytes=0) == RT_EINVAL  # only ws missing


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), RT_EINVAL, "null"),
    (dict(window=0), RT_EINVAL, "window"),
    (dict(d=100), RT_EUNSUPPORTED, "d=100"),
    (dict(out=FAKE), RT_EINVAL, "alias"),
    (dict(causal=-1), RT_EINVAL, "causal"),
    (dict(out_dtype=2), RT_EUNSUPPORTED, "out_dtype"),
])
def test_local_validation(lib, kw, code, msg):
    a = dict(q=FAKE, kk=FAKE, v=FAKE, dtype=1, B=1, H=1, n=64, d=16, window=8, scale=0.25,
             causal=1, out=ctypes.c_void_p(0x2000), out_dtype=1)
    a.update(kw)
    assert lib.rt_local_attn(a["q"], a["kk"], a["v"], a["dtype"], a["B"], a["H"], a["n"], a["d"],
                             a["window"], a["scale"], a["causal"], a["out"], a["out_dtype"],
                             None) == code
    assert msg in _last(lib)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(mu=None), RT_EINVAL, "null"),
    (dict(q_inv=None), RT_EINVAL, "null"),
    (dict(kk=FAKE), RT_EINVAL, "both"),
    (dict(lam=1.5), RT_EINVAL, "lambda"),
    (dict(lam=-0.1), RT_EINVAL, "lambda"),
    (dict(lam=float("nan")), RT_EINVAL, "lambda"),
    (dict(w=100), RT_EINVAL, "exceeds n"),
])
def test_centroid_update_validation(lib, kw, code, msg):
    a = dict(mu=FAKE, q=FAKE, q_inv=FAKE, kk=None, k_inv=None, dtype=1, idx=FAKE, B=1, H=1, n=64,
             d=16, k=4, w=16, lam=0.999)
    a.update(kw)
    assert lib.rt_centroid_update(a["mu"], a["q"], a["q_inv"], a["kk"], a["k_inv"], a["dtype"],
                                  a["idx"], a["B"], a["H"], a["n"], a["d"], a["k"], a["w"],
                                  a["lam"], None) == code
    assert msg in _last(lib)


@pytest.mark.parametrize("args,code,msg", [
    (dict(mu=None), RT_EINVAL, "null"),
    (dict(sq=None), RT_EINVAL, "null"),
    (dict(B=0), RT_EINVAL, "positive"),
    (dict(lam=2.0), RT_EINVAL, "lambda"),
])
def test_centroid_update_sums_validation(lib, args, code, msg):
    a = dict(mu=FAKE, sq=FAKE, sk=None, B=1, H=1, k=4, d=16, lam=0.5)
    a.update(args)
    assert lib.rt_centroid_update_sums(a["mu"], a["sq"], a["sk"], a["B"], a["H"], a["k"], a["d"],
                                       a["lam"], None) == code
    assert msg in _last(lib)


def test_workspace_sizes(lib):
    B, H, n, d, k, w = 1, 8, 8192, 128, 64, 128
    assert lib.rt_workspace_bytes(0, B, H, n, d, k, w) == B * H * k * n * 4
    mask = ((B * H * n * 2 * 4 + 255) // 256) * 256
    slots = ((B * H * n * 4 * d * 4 + 255) // 256) * 256
    dirs = B * H * n * (k - 4) * 4                       # overflow directory
    assert lib.rt_workspace_bytes(1, B, H, n, d, k, w) == mask + slots + B * H * k * w * d * 4 + dirs
    assert lib.rt_workspace_bytes(1, B, H, n, d, 4, w) == (
        ((B * H * n * 4 + 255) // 256) * 256 + slots + B * H * 4 * w * d * 4)   # k <= 4: none
    assert lib.rt_workspace_bytes(2, B, H, n, d, k, w) == 0
    assert lib.rt_workspace_bytes(3, B, H, n, d, k, w) == 0
    assert lib.rt_workspace_bytes(10, B, H, n, d, k, w) == ctypes.c_size_t(-1).value
    assert lib.rt_workspace_bytes(0, 0, H, n, d, k, w) == ctypes.c_size_t(-1).value


def test_binding_rejects_cpu_tensors():
    import torch
    import content_sparse_attention_unit_amd as rt
    x = torch.zeros(1, 1, 64, 16)
    with pytest.raises(ValueError):
        rt.local_attn(x, x, x, 8)


def bwd(lib, q=FAKE, kk=FAKE, v=FAKE, dtype=1, q_inv=FAKE, k_inv=FAKE, idx=FAKE, mask=None,
        lse=ctypes.c_void_p(0x4000), dout=ctypes.c_void_p(0x5000), B=1, H=1, n=64, d=16, k=4,
        w=16, scale=0.25, causal=1, dq=ctypes.c_void_p(0x6000), dk=ctypes.c_void_p(0x7000),
        dv=ctypes.c_void_p(0x8000), ws=None, ws_bytes=0):
    return lib.rt_routed_attn_bwd(q, kk, v, dtype, q_inv, k_inv, idx, mask, lse, dout, B, H, n,
                                  d, k, w, scale, causal, dq, dk, dv, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(lse=None), RT_EINVAL, "null"),
    (dict(dout=None), RT_EINVAL, "null"),
    (dict(dv=None), RT_EINVAL, "null"),
    (dict(q_inv=None), RT_EINVAL, "both"),
    (dict(dq=FAKE), RT_EINVAL, "aliases an input"),
    (dict(dk=ctypes.c_void_p(0x6000)), RT_EINVAL, "alias each other"),
    (dict(q=ctypes.c_void_p(0x3000), dk=None), RT_EINVAL, "only with shared"),
    (dict(dk=None), RT_EINVAL, "workspace"),      # shared q/k: dk may be NULL
    (dict(w=65), RT_EINVAL, "exceeds n"),
    (dict(d=24), RT_EUNSUPPORTED, "d=24"),
    (dict(causal=3), RT_EINVAL, "causal"),
    (dict(scale=float("nan")), RT_EINVAL, "scale"),
    (dict(n=4096, d=128, w=129), RT_EUNSUPPORTED, "w=129"),
    (dict(n=4096, d=64, w=257), RT_EUNSUPPORTED, "w=257"),
    (dict(q=ctypes.c_void_p(0x3000), n=4096, d=64, w=129), RT_EUNSUPPORTED, "w=129"),
    (dict(dtype=0, w=65, n=100), RT_EUNSUPPORTED, "w=65"),
    (dict(), RT_EINVAL, "workspace"),
])
def test_routed_attn_bwd_validation(lib, kw, code, msg):
    assert bwd(lib, **kw) == code
    assert msg in _last(lib)


def test_bwd_workspace_size(lib):
    B, H, n, d, k, w = 1, 8, 32768, 64, 128, 256
    mask = ((B * H * n * 4 * 4 + 255) // 256) * 256
    slots = ((B * H * n * 4 * d * 4 + 255) // 256) * 256
    ovf = B * H * k * w * d * 4
    dirs = ((B * H * n * (k - 4) * 4 + 255) // 256) * 256
    assert lib.rt_workspace_bytes(4, B, H, n, d, k, w) == mask + dirs + 3 * (slots + ovf)


def in_proj(lib, x=FAKE, w=ctypes.c_void_p(0x9000), B=1, n=64, dm=64, d=16, R=2, L=1,
            outs=(0xa000, 0xb000, 0xc000, 0xd000, 0xe000)):
    o = [None if p is None else ctypes.c_void_p(p) for p in outs]
    return lib.rt_in_proj(x, w, B, n, dm, d, R, L, *o, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(x=None), RT_EINVAL, "null"),
    (dict(outs=(0xa000, 0xb000, None, 0xd000, 0xe000)), RT_EINVAL, "local-head output"),
    (dict(outs=(0xa000, 0xa000, 0xc000, 0xd000, 0xe000)), RT_EINVAL, "alias each other"),
    (dict(outs=(0x1000, 0xb000, 0xc000, 0xd000, 0xe000)), RT_EINVAL, "aliases an input"),
    (dict(R=0), RT_EINVAL, "positive"),
    (dict(L=-1), RT_EINVAL, "positive"),
    (dict(d=24), RT_EUNSUPPORTED, "d=24"),
    (dict(dm=60), RT_EUNSUPPORTED, "multiple of 8"),
    (dict(B=4096, n=4096, dm=1024), RT_EUNSUPPORTED, "too large"),
])
def test_in_proj_validation(lib, kw, code, msg):
    assert in_proj(lib, **kw) == code
    assert msg in _last(lib)


def test_in_proj_without_local_heads_needs_no_local_outputs(lib):
    # L = 0: the local outputs may be NULL (fails later only on the fake sizes' check)
    assert in_proj(lib, L=0, outs=(0xa000, 0xb000, None, None, None), d=24) == RT_EUNSUPPORTED


@pytest.mark.parametrize("kw,code,msg", [
    (dict(o_r=None), RT_EINVAL, "null"),
    (dict(o_l=None), RT_EINVAL, "null"),
    (dict(y=0x3000), RT_EINVAL, "aliases"),
    (dict(dm=12), RT_EUNSUPPORTED, "multiple of 8"),
    (dict(d=8), RT_EUNSUPPORTED, "d=8"),
])
def test_out_proj_validation(lib, kw, code, msg):
    a = dict(o_r=0x3000, o_l=0x4000, w_o=0x5000, x=0x6000, B=1, n=64, dm=64, d=16, R=2, L=1,
             y=0x7000)
    a.update(kw)
    p = {k_: (None if a[k_] is None else ctypes.c_void_p(a[k_]))
         for k_ in ("o_r", "o_l", "w_o", "x", "y")}
    assert lib.rt_out_proj(p["o_r"], p["o_l"], p["w_o"], p["x"], a["B"], a["n"], a["dm"], a["d"],
                           a["R"], a["L"], p["y"], None) == code
    assert msg in _last(lib)


# ---- the layer's backward ---------------------------------------------------------------

def lbwd(lib, q=FAKE, kk=ctypes.c_void_p(0x2000), v=ctypes.c_void_p(0x3000),
         dout=ctypes.c_void_p(0x4000), dtype=1, B=1, H=1, n=64, d=64, window=8, scale=0.25,
         causal=1, dq=ctypes.c_void_p(0x6000), dk=ctypes.c_void_p(0x7000),
         dv=ctypes.c_void_p(0x8000), ws=None, ws_bytes=0):
    return lib.rt_local_attn_bwd(q, kk, v, dout, dtype, B, H, n, d, window, scale, causal, dq, dk,
                                 dv, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dout=None), RT_EINVAL, "null"),
    (dict(dk=None), RT_EINVAL, "null"),
    (dict(dq=FAKE), RT_EINVAL, "aliases an input"),
    (dict(dv=ctypes.c_void_p(0x6000)), RT_EINVAL, "alias each other"),
    (dict(window=0), RT_EINVAL, "window"),
    (dict(causal=2), RT_EINVAL, "causal"),
    (dict(scale=float("inf")), RT_EINVAL, "scale"),
    (dict(d=32), RT_EUNSUPPORTED, "d in {64, 128}"),
    (dict(dtype=0), RT_EUNSUPPORTED, "bf16"),
    (dict(d=48), RT_EUNSUPPORTED, "d=48"),
    (dict(), RT_EINVAL, "workspace"),
    (dict(ws=FAKE, ws_bytes=64 * 8 - 1), RT_EINVAL, "workspace"),
])
def test_local_attn_bwd_validation(lib, kw, code, msg):
    assert lbwd(lib, **kw) == code
    assert msg in _last(lib)


def test_local_bwd_workspace_size(lib):
    assert lib.rt_workspace_bytes(5, 2, 4, 1000, 64, 1, 1) == 2 * 4 * 1000 * 8


@pytest.mark.parametrize("kw,code,msg", [
    (dict(x=None), RT_EINVAL, "null"),
    (dict(g1=None), RT_EINVAL, "null"),
    (dict(rows=0), RT_EINVAL, "positive"),
    (dict(d=24), RT_EUNSUPPORTED, "d=24"),
    (dict(dtype=7), RT_EUNSUPPORTED, "dtype"),
    (dict(dx=FAKE), RT_EINVAL, "aliases"),
])
def test_normalize_bwd_validation(lib, kw, code, msg):
    a = dict(x=FAKE, dtype=1, inv=ctypes.c_void_p(0x2000), g1=ctypes.c_void_p(0x3000), g2=None,
             rows=10, d=64, dx=ctypes.c_void_p(0x4000))
    a.update(kw)
    assert lib.rt_normalize_bwd(a["x"], a["dtype"], a["inv"], a["g1"], a["g2"], a["rows"], a["d"],
                                a["dx"], None) == code
    assert msg in _last(lib)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dy=None), RT_EINVAL, "null"),
    (dict(do_l=None), RT_EINVAL, "null"),
    (dict(dw_o=None), RT_EINVAL, "null"),
    (dict(R=0), RT_EINVAL, "positive"),
    (dict(dm=12), RT_EUNSUPPORTED, "multiple of 8"),
    (dict(do_r=FAKE), RT_EINVAL, "aliases an input"),
    (dict(do_l=ctypes.c_void_p(0x5000)), RT_EINVAL, "alias each other"),
])
def test_out_proj_bwd_validation(lib, kw, code, msg):
    a = dict(dy=FAKE, o_r=ctypes.c_void_p(0x2000), o_l=ctypes.c_void_p(0x3000),
             w_o=ctypes.c_void_p(0x4000), B=1, n=16, dm=64, d=16, R=2, L=1,
             do_r=ctypes.c_void_p(0x5000), do_l=ctypes.c_void_p(0x6000),
             dw_o=ctypes.c_void_p(0x7000))
    a.update(kw)
    assert lib.rt_out_proj_bwd(a["dy"], a["o_r"], a["o_l"], a["w_o"], a["B"], a["n"], a["dm"],
                               a["d"], a["R"], a["L"], a["do_r"], a["do_l"], a["dw_o"], None, 0,
                               None) == code
    assert msg in _last(lib)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(x=None), RT_EINVAL, "null"),
    (dict(dv=None), RT_EINVAL, "null"),
    (dict(dk_l=None), RT_EINVAL, "null"),
    (dict(d=40), RT_EUNSUPPORTED, "d=40"),
    (dict(dx=FAKE), RT_EINVAL, "aliases an input"),
    (dict(dw_in=ctypes.c_void_p(0x9000)), RT_EINVAL, "alias"),
])
def test_in_proj_bwd_validation(lib, kw, code, msg):
    a = dict(x=FAKE, w_in=ctypes.c_void_p(0x2000), dqk=ctypes.c_void_p(0x3000),
             dv=ctypes.c_void_p(0x4000), dq_l=ctypes.c_void_p(0x5000),
             dk_l=ctypes.c_void_p(0x6000), dv_l=ctypes.c_void_p(0x7000), dres=None, B=1, n=16,
             dm=64, d=16, R=2, L=1, dx=ctypes.c_void_p(0x9000), dw_in=ctypes.c_void_p(0xa000))
    a.update(kw)
    assert lib.rt_in_proj_bwd(a["x"], a["w_in"], a["dqk"], a["dv"], a["dq_l"], a["dk_l"],
                              a["dv_l"], a["dres"], a["B"], a["n"], a["dm"], a["d"], a["R"],
                              a["L"], a["dx"], a["dw_in"], None, 0, None) == code
    assert msg in _last(lib)


def decode_routed(lib, qk_t=FAKE, v_t=FAKE, mu=FAKE, B=1, H=2, d=64, k=8, cap=64, ck=FAKE,
                  cinv=FAKE, cv=FAKE, cpos=FAKE, clen=FAKE, t=10, scale=0.125, out=FAKE,
                  out_dtype=0, label=None):
    return lib.rt_decode_routed(qk_t, v_t, mu, B, H, d, k, cap, ck, cinv, cv, cpos, clen, t,
                                ctypes.c_float(scale), out, out_dtype, label, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(qk_t=None), RT_EINVAL, "null"),
    (dict(clen=None), RT_EINVAL, "null"),
    (dict(out=None), RT_EINVAL, "null"),
    (dict(B=0), RT_EINVAL, "positive"),
    (dict(d=48), RT_EUNSUPPORTED, "d=48"),
    (dict(k=0), RT_EINVAL, "k=0"),
    (dict(k=257), RT_EUNSUPPORTED, "exceeds 256"),
    (dict(cap=0), RT_EINVAL, "cap=0"),
    (dict(cap=16385), RT_EUNSUPPORTED, "exceeds 16384"),
    (dict(t=-1), RT_EINVAL, "negative"),
    (dict(scale=float("inf")), RT_EINVAL, "scale"),
    (dict(out_dtype=3), RT_EUNSUPPORTED, "out_dtype"),
    (dict(B=300, H=300), RT_EUNSUPPORTED, "B*H"),
])
def test_decode_routed_validation(lib, kw, code, msg):
    assert decode_routed(lib, **kw) == code
    assert msg in _last(lib)


def decode_local(lib, q_t=FAKE, k_t=FAKE, v_t=FAKE, B=1, H=2, d=64, window=32, rk=FAKE, rv=FAKE,
                 t=0, scale=0.125, out=FAKE, out_dtype=1):
    return lib.rt_decode_local(q_t, k_t, v_t, B, H, d, window, rk, rv, t, ctypes.c_float(scale),
                               out, out_dtype, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(rk=None), RT_EINVAL, "null"),
    (dict(H=0), RT_EINVAL, "positive"),
    (dict(d=256), RT_EUNSUPPORTED, "d=256"),
    (dict(window=0), RT_EINVAL, "window=0"),
    (dict(window=20000), RT_EUNSUPPORTED, "exceeds 16384"),
    (dict(t=-5), RT_EINVAL, "negative"),
    (dict(scale=float("nan")), RT_EINVAL, "scale"),
    (dict(out_dtype=2), RT_EUNSUPPORTED, "out_dtype"),
])
def test_decode_local_validation(lib, kw, code, msg):
    assert decode_local(lib, **kw) == code
    assert msg in _last(lib)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(idx=None), RT_EINVAL, "null"),
    (dict(w=0), RT_EINVAL, "positive"),
    (dict(w=65), RT_EINVAL, "exceeds n"),
    (dict(cap=15), RT_EINVAL, "below w"),
    (dict(cap=20000), RT_EUNSUPPORTED, "exceeds 16384"),
    (dict(d=24), RT_EUNSUPPORTED, "d=24"),
])
def test_decode_fill_validation(lib, kw, code, msg):
    a = dict(qk=FAKE, inv=FAKE, v=FAKE, idx=FAKE, B=1, H=1, n=64, d=16, k=4, w=16, cap=32)
    a.update(kw)
    assert lib.rt_decode_fill(a["qk"], a["inv"], a["v"], a["idx"], a["B"], a["H"], a["n"], a["d"],
                              a["k"], a["w"], a["cap"], FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
    assert msg in _last(lib)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(kk=None), RT_EINVAL, "null"),
    (dict(n=0), RT_EINVAL, "positive"),
    (dict(window=0), RT_EINVAL, "window=0"),
])
def test_decode_ring_fill_validation(lib, kw, code, msg):
    a = dict(kk=FAKE, B=1, H=1, n=64, d=16, window=8)
    a.update(kw)
    assert lib.rt_decode_ring_fill(a["kk"], FAKE, a["B"], a["H"], a["n"], a["d"], a["window"],
                                   FAKE, FAKE, None) == code
    assert msg in _last(lib)


def test_decode_binding_rejects_float32_rows():
    import torch
    import content_sparse_attention_unit_amd as rt
    with pytest.raises((TypeError, ValueError)):
        rt.decode_local(*(torch.zeros(1, 1, 4, 16) for _ in range(2)),
                        *(torch.zeros(1, 1, 16) for _ in range(3)), 0)


def attn_split(lib, q=FAKE, kk=ctypes.c_void_p(0x3000), v=FAKE, dtype=1, idx_q=FAKE, idx_k=FAKE,
               n=64, d=16, k=4, w=16, out=ctypes.c_void_p(0x2000), ws=FAKE, ws_bytes=0):
    return lib.rt_routed_attn_split(q, kk, v, dtype, FAKE, FAKE, idx_q, idx_k, None, 1, 1, n, d,
                                    k, w, 0.25, out, 1, None, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(idx_q=None), RT_EINVAL, "null"),
    (dict(idx_k=None), RT_EINVAL, "null"),
    (dict(w=65), RT_EINVAL, "exceeds n"),
    (dict(n=4096, d=128, w=200), RT_EUNSUPPORTED, "w=200"),
    (dict(out=FAKE), RT_EINVAL, "alias"),
    (dict(), RT_EINVAL, "workspace"),
])
def test_routed_attn_split_validation(lib, kw, code, msg):
    assert attn_split(lib, **kw) == code
    assert msg in _last(lib)


def attn_js(lib, qk=FAKE, q_inv=FAKE, idx=FAKE, n=64, d=16, k=4, w=16, window=8, causal=1,
            js=ctypes.c_void_p(0x2000), ws=FAKE, ws_bytes=0):
    return lib.rt_attn_js(qk, q_inv, idx, FAKE, FAKE, 1, 1, n, d, k, w, window, 0.25, 0.25,
                          causal, js, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(qk=None), RT_EINVAL, "null"),
    (dict(js=None), RT_EINVAL, "null"),
    (dict(w=65), RT_EINVAL, "exceeds n"),
    (dict(n=4096, d=128, w=200), RT_EUNSUPPORTED, "w=200"),
    (dict(d=48), RT_EUNSUPPORTED, "d=48"),
    (dict(window=0), RT_EINVAL, "window"),
    (dict(causal=3), RT_EINVAL, "causal"),
    (dict(), RT_EINVAL, "workspace"),
])
def test_attn_js_validation(lib, kw, code, msg):
    assert attn_js(lib, **kw) == code
    assert msg in _last(lib)


def test_attn_js_workspace_size(lib):
    assert lib.rt_workspace_bytes(8, 1, 2, 100, 64, 4, 25) == 25600 + 1024


def attn_update(lib, mu=FAKE, lam=0.9, ws=FAKE, ws_bytes=1 << 40):
    return lib.rt_routed_attn_update(FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, 1, 1, 64, 16, 4,
                                     16, 0.25, 1, ctypes.c_void_p(0x2000), 1, None, mu,
                                     ctypes.c_float(lam), ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(mu=None), RT_EINVAL, "null"),
    (dict(lam=1.5), RT_EINVAL, "lambda"),
    (dict(lam=float("nan")), RT_EINVAL, "lambda"),
    (dict(ws_bytes=100), RT_EINVAL, "workspace"),
])
def test_routed_attn_update_validation(lib, kw, code, msg):
    assert attn_update(lib, **kw) == code
    assert msg in _last(lib)


def test_routed_attn_update_workspace_size(lib):
    plain = lib.rt_workspace_bytes(1, 2, 3, 100, 64, 8, 20)
    assert lib.rt_workspace_bytes(9, 2, 3, 100, 64, 8, 20) == plain + 2 * 2 * 3 * 8 * 64 * 4


def test_proj_bwd_workspace_size(lib):
    # the long stack layer: dW_o (1024 x 1536, 96 output tiles) splits 5 ways over 8192
    # tokens, dW_in (3584 x 1024, 224 tiles) 2 ways: the larger of the two partial sets
    B, n, dm, d, R, L = 1, 8192, 1024, 128, 8, 4
    want = max(5 * dm * (R + L) * d * 4, 2 * (2 * R + 3 * L) * d * dm * 4)
    assert lib.rt_proj_bwd_workspace_bytes(B, n, dm, d, R, L) == want
    assert lib.rt_proj_bwd_workspace_bytes(1, 64, 64, 16, 2, 1) == 0     # too few k-tiles
    assert lib.rt_proj_bwd_workspace_bytes(0, 64, 64, 16, 2, 1) == ctypes.c_size_t(-1).value
