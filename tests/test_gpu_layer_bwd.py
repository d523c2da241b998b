"""GPU parity of the layer's backward (rt_local_attn_bwd, rt_normalize_bwd,
rt_out_proj_bwd, rt_in_proj_bwd and their composition with
rt_routed_attn_bwd) against the fp64 oracle, on the same seeded inputs.

Rules.  Attention gradients (bf16 inputs, P and dl rounded to bf16 for the
products): max-abs <= 2e-2 * max(1, max|oracle|) and mean-rel <= 5e-3, as for
the routed backward.  The normalisation's gradient is float32 arithmetic:
within 1e-5 * max(1, |oracle|) elementwise.  The projections' products take
bf16 operands (the oracle rounds the same operands) with float32 accumulation:
each element within the float32 summation bound K * 2^-24 * sum_k |a_k b_k|
(plus one bf16 unit in the last place where the result is stored in bf16).
The whole layer: the oracle's backward on the GPU forward's own values,
gradients within the attention rule.
"""
import math
import sys

import numpy as np
import pytest
import torch

import synthetic as S
from _util import BF16_MAX_ABS, BF16_MEAN_REL, dev_tensor, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import content_sparse_attention_unit_amd as m
    m._load()
    return m


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_grad_close(got, want, what):
    err = np.abs(np.asarray(got, np.float64) - want)
    mag = max(1.0, float(np.abs(want).max()))
    at = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= BF16_MAX_ABS * mag, (f"{what}: max-abs {err.max():.3e} at {at}: got "
                                            f"{got[at]:.6g} want {want[at]:.6g}")
    mean_rel = err.sum() / max(np.abs(want).sum(), 1e-30)
    assert mean_rel <= BF16_MEAN_REL, f"{what}: mean-rel {mean_rel:.3e}"


def assert_within(got, want, bound, what, bf16_out=False):
    got = np.asarray(got, np.float64)
    tol = bound + 2.0 ** -23 * np.abs(want)        # the float32 result's own rounding
    if bf16_out:
        a = np.abs(want)
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        tol = tol + np.where(a > 0, np.ldexp(1.0, (e - 7).astype(int)), 0.0)
    bad = np.abs(got - want) > tol
    if bad.any():
        at = np.unravel_index(np.argmax(np.where(bad, np.abs(got - want) - tol, 0)), got.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} beyond the bound, at {at}: got "
                             f"{got[at]!r} want {want[at]!r} tol {tol[at]:.3e}")


# ---- local attention backward ----------------------------------------------------------

LOCAL = {
    # name: (B, H, n, d, window, causal)
    "d64_ragged": (1, 2, 300, 64, 50, True),
    "d128_ragged": (2, 1, 257, 128, 64, True),
    "window1": (1, 1, 200, 64, 1, True),
    "window_gt_n": (1, 1, 130, 128, 500, True),
    "non_causal": (1, 2, 333, 64, 40, False),
    "d128_w512": (1, 1, 1000, 128, 512, True),
}


def local_inputs(seed, B, H, n, d):
    return [S.normal_tensor(seed + i, (B, H, n, d), "bf16") for i in range(4)]


@pytest.mark.parametrize("name", list(LOCAL))
def test_local_attn_bwd(rt, orc, name):
    B, H, n, d, window, causal = LOCAL[name]
    say(f"[case] local_attn_bwd {name}")
    seed = 70_000 + 10 * list(LOCAL).index(name)
    q, kk, v, g = local_inputs(seed, B, H, n, d)
    sc = 1.0 / math.sqrt(d)
    got = rt.local_attn_bwd(*(dev_tensor(t) for t in (q, kk, v, g)), window, scale=sc,
                            causal=causal)
    torch.cuda.synchronize()
    want = orc.local_attn_bwd(q.value, kk.value, v.value, g.value, window, sc, causal)
    for nm, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_grad_close(host(a), b, f"{name} {nm}")


def test_local_attn_bwd_full_size(rt, orc):
    """The long workload's local heads (n=8192, window 512, d=128), all four, in
    the launch configuration the benchmark times."""
    cfg = S.CONFIGS["long"]
    say("[case] local_attn_bwd long")
    inp = S.make_inputs(cfg)
    g = S.normal_tensor(1000 * cfg.cfg_id + 50, (cfg.B, cfg.L, cfg.n, cfg.d), "bf16")
    sc = 1.0 / math.sqrt(cfg.d)
    got = rt.local_attn_bwd(dev_tensor(inp["q_local"]), dev_tensor(inp["k_local"]),
                            dev_tensor(inp["v_local"]), dev_tensor(g), cfg.window, scale=sc)
    torch.cuda.synchronize()
    want = orc.local_attn_bwd(inp["q_local"].value, inp["k_local"].value, inp["v_local"].value,
                              g.value, cfg.window, sc, True)
    for nm, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_grad_close(host(a), b, f"long {nm}")


def test_local_attn_bwd_deterministic(rt):
    B, H, n, d, window, causal = LOCAL["d64_ragged"]
    ts = [dev_tensor(t) for t in local_inputs(70_900, B, H, n, d)]
    a = rt.local_attn_bwd(*ts, window)
    b = rt.local_attn_bwd(*ts, window)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---- normalisation backward ------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 32), ("bf16", 16)])
def test_normalize_bwd(rt, orc, dtype, d):
    say(f"[case] normalize_bwd {dtype} d={d}")
    x = S.normal_tensor(71_000 + d, (2, 3, 100, d), dtype)
    xv = x.value.copy()
    xd = dev_tensor(x)
    xd[1, 2, 7] = 0                                   # a zero row: the clamped branch
    xv[1, 2, 7] = 0.0
    g1 = S.normal(71_100 + d, (2, 3, 100, d)).astype(np.float32)
    g2 = S.normal(71_200 + d, (2, 3, 100, d)).astype(np.float32)
    inv = torch.from_numpy(
        (1.0 / np.maximum(np.sqrt((xv * xv).sum(-1)), 1e-12)).astype(np.float32)).cuda()
    got = rt.normalize_bwd(xd, inv, torch.from_numpy(g1).cuda(), torch.from_numpy(g2).cuda())
    got1 = rt.normalize_bwd(xd, inv, torch.from_numpy(g1).cuda())
    torch.cuda.synchronize()
    for res, g in ((got, g1.astype(np.float64) + g2), (got1, g1.astype(np.float64))):
        want = orc.normalize_bwd(xv, g)
        h = host(res)
        rel = np.abs(h - want) / np.maximum(1.0, np.abs(want))
        assert rel.max() <= 1e-5, f"max rel {rel.max():.3e}"


# ---- projections' backward ---------------------------------------------------------------

PROJ = {
    # name: (B, n, dm, d, R, L)
    "ragged_d64": (2, 300, 256, 64, 2, 1),
    "d16": (1, 200, 64, 16, 3, 2),
    "no_local": (1, 130, 96, 32, 2, 0),
    "d128": (1, 256, 512, 128, 2, 1),
    # enough tokens for the weight gradients to split their contraction (ragged last split)
    "split_ragged": (1, 2500, 192, 64, 2, 1),
    "split_b2": (2, 1024, 256, 64, 2, 1),
}


def proj_bwd_case(B, n, dm, d, R, L, seed):
    x = S.normal_tensor(seed, (B, n, dm), "bf16")
    w_in = S.normal_tensor(seed + 1, ((2 * R + 3 * L) * d, dm), "bf16", sigma=1 / math.sqrt(dm))
    w_o = S.normal_tensor(seed + 2, (dm, (R + L) * d), "bf16", sigma=1 / math.sqrt((R + L) * d))
    o_r = S.normal_tensor(seed + 3, (B, R, n, d), "bf16")
    o_l = S.normal_tensor(seed + 4, (B, L, n, d), "bf16") if L > 0 else None
    dy = S.normal_tensor(seed + 5, (B, n, dm), "bf16")
    dc = [S.normal(seed + 6 + i, (B, h, n, d)).astype(np.float32).astype(np.float64)
          for i, h in enumerate((R, R, L, L, L)) if h > 0]
    return x, w_in, w_o, o_r, o_l, dy, dc


def check_out_proj_bwd(rt, orc, x, w_in, w_o, o_r, o_l, dy, rows=None):
    got = rt.out_proj_bwd(dev_tensor(dy), dev_tensor(o_r),
                          None if o_l is None else dev_tensor(o_l), dev_tensor(w_o))
    torch.cuda.synchronize()
    sel = (lambda a: a) if rows is None else (lambda a: a[:, :, rows])
    dyv = dy.value if rows is None else dy.value[:, rows]
    do_r, do_l, dw_o = orc.out_proj_bwd(dyv, sel(o_r.value),
                                        None if o_l is None else sel(o_l.value), w_o.value)
    a_r, a_l, _ = orc.out_proj_bwd(np.abs(dyv), sel(np.abs(o_r.value)),
                                   None if o_l is None else sel(np.abs(o_l.value)),
                                   np.abs(w_o.value), rounding=False)
    K = w_o.shape[0] if hasattr(w_o, "shape") else w_o.value.shape[0]
    kb = 1.01 * K * 2.0 ** -24
    assert_within(sel(host(got[0])), do_r, kb * a_r, "do_r", bf16_out=True)
    if o_l is not None:
        assert_within(sel(host(got[1])), do_l, kb * a_l, "do_l", bf16_out=True)
    if rows is None:
        _, _, m_w = orc.out_proj_bwd(np.abs(dy.value), np.abs(o_r.value),
                                     None if o_l is None else np.abs(o_l.value), np.abs(w_o.value),
                                     rounding=False)
        T = dy.value.shape[0] * dy.value.shape[1]
        assert_within(host(got[2]), dw_o, 1.01 * T * 2.0 ** -24 * m_w, "dw_o")


def check_in_proj_bwd(rt, orc, x, w_in, dy, dc, R, L, d, with_res=True):
    dcd = [torch.from_numpy(a.astype(np.float32)).cuda() for a in dc]
    loc = dcd[2:] if L > 0 else [None, None, None]
    dx, dw_in = rt.in_proj_bwd(dev_tensor(x), dev_tensor(w_in), dcd[0], dcd[1], *loc,
                               dres=dev_tensor(dy) if with_res else None)
    torch.cuda.synchronize()
    loc_o = dc[2:] if L > 0 else [None, None, None]
    want_dx, want_dw = orc.in_proj_bwd(x.value, w_in.value, dc[0], dc[1], *loc_o,
                                       dy=dy.value if with_res else None)
    rnd = [orc.round_bf16(a) for a in dc]
    loc_a = [np.abs(a) for a in rnd[2:]] if L > 0 else [None, None, None]
    m_dx, m_dw = orc.in_proj_bwd(np.abs(x.value), np.abs(w_in.value), np.abs(rnd[0]),
                                 np.abs(rnd[1]), *loc_a, rounding=False)
    K = (2 * R + 3 * L) * d
    T = x.value.shape[0] * x.value.shape[1]
    bound_dx = 1.01 * (K + 1) * 2.0 ** -24 * (m_dx + (np.abs(dy.value) if with_res else 0.0))
    assert_within(host(dx), want_dx, bound_dx, "dx")
    assert_within(host(dw_in), want_dw, 1.01 * T * 2.0 ** -24 * m_dw, "dw_in")


@pytest.mark.parametrize("name", list(PROJ))
def test_out_proj_bwd(rt, orc, name):
    B, n, dm, d, R, L = PROJ[name]
    say(f"[case] out_proj_bwd {name}")
    x, w_in, w_o, o_r, o_l, dy, dc = proj_bwd_case(B, n, dm, d, R, L,
                                                   72_000 + 20 * list(PROJ).index(name))
    check_out_proj_bwd(rt, orc, x, w_in, w_o, o_r, o_l, dy)


@pytest.mark.parametrize("name", list(PROJ))
@pytest.mark.parametrize("with_res", [True, False])
def test_in_proj_bwd(rt, orc, name, with_res):
    B, n, dm, d, R, L = PROJ[name]
    say(f"[case] in_proj_bwd {name} res={with_res}")
    x, w_in, w_o, o_r, o_l, dy, dc = proj_bwd_case(B, n, dm, d, R, L,
                                                   73_000 + 20 * list(PROJ).index(name))
    check_in_proj_bwd(rt, orc, x, w_in, dy, dc, R, L, d, with_res)


def test_proj_bwd_full_size(rt, orc):
    """The long stack's shapes (n=8192, d_model=1024, 8 + 4 heads of 128): all
    of dw_o, dw_in and dx, and do on 256 sampled tokens."""
    sc = S.STACKS["long_stack"]
    say("[case] proj bwd long")
    x, w_in, w_o, o_r, o_l, dy, dc = proj_bwd_case(sc.B, sc.n, sc.dm, sc.d, sc.R, sc.L, 74_000)
    check_in_proj_bwd(rt, orc, x, w_in, dy, dc, sc.R, sc.L, sc.d)
    got = rt.out_proj_bwd(dev_tensor(dy), dev_tensor(o_r), dev_tensor(o_l), dev_tensor(w_o))
    torch.cuda.synchronize()
    _, _, dw_o = orc.out_proj_bwd(dy.value, o_r.value, o_l.value, w_o.value)
    _, _, m_w = orc.out_proj_bwd(np.abs(dy.value), np.abs(o_r.value), np.abs(o_l.value),
                                 np.abs(w_o.value), rounding=False)
    assert_within(host(got[2]), dw_o, 1.01 * sc.n * 2.0 ** -24 * m_w, "dw_o")
    rows = np.sort(np.random.default_rng(9).choice(sc.n, 256, replace=False))
    check_out_proj_bwd(rt, orc, x, w_in, w_o, o_r, o_l, dy, rows=rows)


def test_weight_grad_split_is_deterministic_and_matches_unsplit(rt, orc):
    """The split weight gradients: bit-identical on repeats, and the unsplit
    products (no workspace) within the same float32 summation bound."""
    B, n, dm, d, R, L = PROJ["split_ragged"]
    x, w_in, w_o, o_r, o_l, dy, dc = proj_bwd_case(B, n, dm, d, R, L, 77_000)
    ws = rt.proj_bwd_workspace(B, n, dm, d, R, L, "cuda")
    assert ws is not None
    args = (dev_tensor(dy), dev_tensor(o_r), dev_tensor(o_l), dev_tensor(w_o))
    a = rt.out_proj_bwd(*args, ws=ws)[2].clone()
    b = rt.out_proj_bwd(*args, ws=ws)[2].clone()
    c = rt.out_proj_bwd(*args, ws=None)[2]
    dcd = [torch.from_numpy(t.astype(np.float32)).cuda() for t in dc]
    xin = (dev_tensor(x), dev_tensor(w_in), *dcd)
    e = rt.in_proj_bwd(*xin, ws=ws)[1].clone()
    f = rt.in_proj_bwd(*xin, ws=ws)[1].clone()
    g = rt.in_proj_bwd(*xin, ws=None)[1]
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(e, f)
    _, _, dw_o = orc.out_proj_bwd(dy.value, o_r.value, o_l.value, w_o.value)
    _, _, m_w = orc.out_proj_bwd(np.abs(dy.value), np.abs(o_r.value), np.abs(o_l.value),
                                 np.abs(w_o.value), rounding=False)
    assert_within(host(c), dw_o, 1.01 * n * 2.0 ** -24 * m_w, "dw_o unsplit")
    _, want_dw = orc.in_proj_bwd(x.value, w_in.value, *dc)
    rnd = [np.abs(orc.round_bf16(t)) for t in dc]
    _, m_dw = orc.in_proj_bwd(np.abs(x.value), np.abs(w_in.value), *rnd, rounding=False)
    assert_within(host(g), want_dw, 1.01 * n * 2.0 ** -24 * m_dw, "dw_in unsplit")


# ---- the whole layer ---------------------------------------------------------------------

LAYERS = {
    "d64": S.StackConfig(75, "bwd_layer_d64", 1, 300, 128, 64, 1, 1, 4, 64, 48, 1),
    "d128_b2": S.StackConfig(76, "bwd_layer_d128", 2, 256, 256, 128, 2, 1, 4, 64, 100, 1),
}


@pytest.mark.parametrize("name", list(LAYERS))
def test_layer_backward(rt, orc, name):
    """GPU forward, then the GPU backward chain; the oracle's layer_backward runs
    on the GPU forward's own values (projections, membership, head outputs)."""
    sc = LAYERS[name]
    say(f"[case] layer backward {name}")
    x = S.stack_x(sc)
    lw = S.stack_layer(sc, 0)
    dy = S.normal_tensor(1000 * sc.cfg_id + 60, (sc.B, sc.n, sc.dm), "bf16")
    scale = 1.0 / math.sqrt(sc.d)
    xd, w_in, w_o = dev_tensor(x), dev_tensor(lw["w_in"]), dev_tensor(lw["w_o"])
    mu = dev_tensor(lw["mu"])
    qk, v, ql, kl, vl = rt.in_proj(xd, w_in, sc.R, sc.L, sc.d)
    inv, idx = rt.route(qk, mu, sc.w)
    o_r, lse = rt.routed_attn(qk, qk, v, idx, inv, inv, scale=scale, want_lse=True)
    o_l = rt.local_attn(ql, kl, vl, sc.window, scale=scale)
    dyd = dev_tensor(dy)
    do_r, do_l, dw_o = rt.out_proj_bwd(dyd, o_r, o_l, w_o)
    dqh, dkh, dv = rt.routed_attn_bwd(qk, qk, v, idx, lse, do_r, inv, inv, scale=scale)
    dqk = rt.normalize_bwd(qk, inv, dqh, dkh)
    dq_l, dk_l, dv_l = rt.local_attn_bwd(ql, kl, vl, do_l, sc.window, scale=scale)
    dx, dw_in = rt.in_proj_bwd(xd, w_in, dqk, dv, dq_l, dk_l, dv_l, dres=dyd)
    torch.cuda.synchronize()

    fwd = {"qk": host(qk), "v": host(v), "q_l": host(ql), "k_l": host(kl), "v_l": host(vl),
           "idx": host(idx), "o_r": host(o_r), "o_l": host(o_l)}
    want = orc.layer_backward(x.value, lw["w_in"].value, lw["w_o"].value, fwd, dy.value, sc.R,
                              sc.L, sc.d, sc.window, scale)
    assert_grad_close(host(do_r), want["do_r"], "do_r")
    assert_grad_close(host(dqk), want["dqk"], "dqk")
    assert_grad_close(host(dq_l), want["dq_l"], "dq_l")
    assert_grad_close(host(dw_o), want["dw_o"], "dw_o")
    assert_grad_close(host(dx), want["dx"], "dx")
    assert_grad_close(host(dw_in), want["dw_in"], "dw_in")
