"""GPU parity of the layer-stack pieces: the projections (rt_in_proj,
rt_out_proj) and one whole layer, against the fp64 oracle.

Rules.  A bfloat16 result is the rounding of a float32 (device) or exact
(oracle) sum of K products, so each element must be within one bfloat16 unit
in the last place plus the float32 summation bound K * 2^-24 * sum_k |a_k w_k|
(which matters only where the sum cancels), and at most 1% of the elements
may differ at all.  In a whole layer the
projections' one-ulp differences move the routing scores by about 1e-4, so
memberships must agree wherever the oracle's margin exceeds 1e-3, and the
layer output is compared on the tokens no differing cluster touches, within
2e-2 * max(1, |oracle|) (mean-rel 5e-3).
"""
import math
import sys

import numpy as np
import pytest
import torch

import synthetic as S
from _util import (BF16_MEAN_REL, MU_MAX_ABS, check_membership, dev_tensor, host,
                   tokens_touched)

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


def ulp_bf16(a):
    a = np.abs(np.asarray(a, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (e - 7).astype(int)), 0.0)


def assert_bf16_rounding_close(got, want, what, bound=0.0, max_frac=0.01):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    diff = np.abs(got - want)
    tol = np.maximum(ulp_bf16(want), ulp_bf16(got)) + bound
    bad = diff > tol
    if bad.any():
        at = np.unravel_index(np.argmax(np.where(bad, diff, 0)), diff.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond one ulp, at {at}: "
                             f"got {got[at]!r} want {want[at]!r}")
    frac = float((diff > 0).mean()) if diff.size else 0.0
    assert frac <= max_frac, f"{what}: {frac:.3%} of elements differ (one ulp each)"


def in_bounds(orc, x, w_in, R, L, d):
    """float32 summation bounds of the five projections (head-major, like them)."""
    K = x.shape[-1]
    mags = orc.in_proj(np.abs(x), np.abs(w_in), R, L, d)
    return [None if m_ is None else 1.01 * K * 2.0 ** -24 * m_ for m_ in mags]


def out_bound(orc, o_r, o_l, w_o, x):
    K = w_o.shape[1]
    m_ = orc.out_proj(np.abs(o_r), None if o_l is None else np.abs(o_l), np.abs(w_o),
                      None if x is None else np.abs(x))
    return 1.01 * (K + 1) * 2.0 ** -24 * m_


def proj_case(B, n, dm, d, R, L, seed):
    x = S.normal_tensor(seed, (B, n, dm), "bf16")
    w_in = S.normal_tensor(seed + 1, ((2 * R + 3 * L) * d, dm), "bf16", sigma=1 / math.sqrt(dm))
    w_o = S.normal_tensor(seed + 2, (dm, (R + L) * d), "bf16", sigma=1 / math.sqrt((R + L) * d))
    o_r = S.normal_tensor(seed + 3, (B, R, n, d), "bf16")
    o_l = S.normal_tensor(seed + 4, (B, L, n, d), "bf16") if L > 0 else None
    return x, w_in, w_o, o_r, o_l


PROJ = {
    "ragged_d64": (2, 300, 256, 64, 2, 1),
    "d16": (1, 200, 64, 16, 3, 2),
    "d32_no_local_k96": (1, 130, 96, 32, 2, 0),
    "d128": (1, 256, 512, 128, 2, 1),
}


@pytest.mark.parametrize("name", list(PROJ))
def test_in_proj(rt, orc, name):
    B, n, dm, d, R, L = PROJ[name]
    say(f"[case] in_proj {name}")
    x, w_in, _, _, _ = proj_case(B, n, dm, d, R, L, 60_000 + 10 * list(PROJ).index(name))
    got = rt.in_proj(dev_tensor(x), dev_tensor(w_in), R, L, d)
    torch.cuda.synchronize()
    want = orc.in_proj(x.value, w_in.value, R, L, d)
    bounds = in_bounds(orc, x.value, w_in.value, R, L, d)
    for nm, g, w_, b_ in zip(("qk", "v", "q_l", "k_l", "v_l"), got, want, bounds):
        if w_ is None:
            assert g is None
            continue
        assert_bf16_rounding_close(host(g), w_, f"in_proj {nm}", b_)


@pytest.mark.parametrize("name", list(PROJ))
@pytest.mark.parametrize("residual", ["x", "none", "in_place"])
def test_out_proj(rt, orc, name, residual):
    B, n, dm, d, R, L = PROJ[name]
    say(f"[case] out_proj {name} residual={residual}")
    x, _, w_o, o_r, o_l = proj_case(B, n, dm, d, R, L, 61_000 + 10 * list(PROJ).index(name))
    xd = dev_tensor(x)
    args = (dev_tensor(o_r), None if o_l is None else dev_tensor(o_l), dev_tensor(w_o))
    if residual == "x":
        y = rt.out_proj(*args, x=xd)
    elif residual == "none":
        y = rt.out_proj(*args)
    else:
        y = rt.out_proj(*args, x=xd, out=xd)
        assert y.data_ptr() == xd.data_ptr()
    torch.cuda.synchronize()
    args_o = (o_r.value, None if o_l is None else o_l.value, w_o.value,
              None if residual == "none" else x.value)
    assert_bf16_rounding_close(host(y), orc.out_proj(*args_o), "out_proj", out_bound(orc, *args_o))


def test_proj_full_size_sampled(rt, orc):
    """Layer 0 of the long stack (n=8192, d_model=1024, 8+4 heads of 128) in the
    benchmark's launch configuration; 256 sampled tokens against the oracle."""
    sc = S.STACKS["long_stack"]
    x = S.stack_x(sc)
    lw = S.stack_layer(sc, 0)
    got = rt.in_proj(dev_tensor(x), dev_tensor(lw["w_in"]), sc.R, sc.L, sc.d)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(7).choice(sc.n, 256, replace=False))
    want = orc.in_proj(x.value[:, rows], lw["w_in"].value, sc.R, sc.L, sc.d)
    bounds = in_bounds(orc, x.value[:, rows], lw["w_in"].value, sc.R, sc.L, sc.d)
    for nm, g, w_, b_ in zip(("qk", "v", "q_l", "k_l", "v_l"), got, want, bounds):
        assert_bf16_rounding_close(host(g)[:, :, rows], w_, f"in_proj {nm}", b_)
    o_r = got[0]
    o_l = got[2]
    y = rt.out_proj(o_r, o_l, dev_tensor(lw["w_o"]), x=dev_tensor(x))
    torch.cuda.synchronize()
    args_o = (host(o_r)[:, :, rows], host(o_l)[:, :, rows], lw["w_o"].value, x.value[:, rows])
    assert_bf16_rounding_close(host(y)[:, rows], orc.out_proj(*args_o), "out_proj",
                               out_bound(orc, *args_o))


def gpu_layer(rt, x, lw, sc, scale):
    qk, v, ql, kl, vl = rt.in_proj(x, lw["w_in"], sc.R, sc.L, sc.d)
    mu = lw["mu"].clone()
    inv, idx = rt.route(qk, mu, sc.w)
    o_r = rt.routed_attn(qk, qk, v, idx, inv, inv, scale=scale)
    rt.centroid_update_(mu, qk, inv, idx, sc.lam)
    o_l = rt.local_attn(ql, kl, vl, sc.window, scale=scale) if sc.L > 0 else None
    y = rt.out_proj(o_r, o_l, lw["w_o"], x=x)
    return dict(qk=qk, v=v, q_l=ql, k_l=kl, v_l=vl, idx=idx, mu=mu, o_r=o_r, o_l=o_l, y=y)


def check_layer(orc, got, want, sc, x, w_in, tau=1e-3):
    bounds = dict(zip(("qk", "v", "q_l", "k_l", "v_l"), in_bounds(orc, x, w_in, sc.R, sc.L, sc.d)))
    for nm in ("qk", "v", "q_l", "k_l", "v_l"):
        if want[nm] is not None:
            assert_bf16_rounding_close(host(got[nm]), want[nm], f"layer {nm}", bounds[nm])
    gidx = host(got["idx"])
    same = (gidx == want["idx"]).all(-1)
    bad = np.argwhere((want["margin"] > tau) & ~same)
    assert bad.size == 0, f"membership differs on {len(bad)} clusters with margin > {tau}"
    keep = ~tokens_touched(gidx, want["idx"], ~same, sc.n)             # [B,R,n]
    keep_tok = keep.all(axis=1)                                         # every routed head
    y, yw = host(got["y"])[keep_tok], want["y"][keep_tok]
    err = np.abs(y - yw)
    assert err.size > 0
    assert np.all(err <= 2e-2 * np.maximum(1.0, np.abs(yw))), f"y: max err {err.max():.3e}"
    assert err.sum() / np.abs(yw).sum() <= BF16_MEAN_REL
    same_c = ~(~same).any(axis=0)
    assert np.abs(host(got["mu"])[same_c] - want["mu"][same_c]).max(initial=0.0) <= MU_MAX_ABS
    return int((~same).sum()), float(keep_tok.mean())


def assert_rows_close(got, want, what):
    """Attention outputs: each element within 2e-2 of the largest magnitude in
    its output row (a row may cancel to near zero where the values it averages
    are large), and mean-rel 5e-3 over the whole tensor."""
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    scale = np.maximum(1.0, np.abs(want).max(axis=-1, keepdims=True))
    err = np.abs(got - want)
    assert np.all(err <= 2e-2 * scale), f"{what}: max scaled err {(err / scale).max():.3e}"
    assert err.sum() / max(np.abs(want).sum(), 1e-300) <= BF16_MEAN_REL, f"{what}: mean-rel"


def check_layer_staged(orc, got, x_in, lw, sc, scale):
    """One layer at any depth, each stage against the oracle run on the device's
    own input to that stage (so that no difference carries over from an earlier
    stage): the five projections within one ulp plus the float32 summation
    bound; memberships by the margin rule on the device's qk; the routed heads
    on the device's membership and the local heads, by the row-scaled rule;
    the centroid update within 1e-5; the layer output, from the device's head
    outputs and the residual, within one ulp plus the summation bound.  Returns
    the number of clusters a near-tie let differ."""
    w_in, w_o, mu0 = lw["w_in"].value, lw["w_o"].value, lw["mu"]
    want5 = orc.in_proj(x_in, w_in, sc.R, sc.L, sc.d)
    bounds = in_bounds(orc, x_in, w_in, sc.R, sc.L, sc.d)
    for nm, w_, b_ in zip(("qk", "v", "q_l", "k_l", "v_l"), want5, bounds):
        if w_ is not None:
            assert_bf16_rounding_close(host(got[nm]), w_, f"layer {nm}", b_)
    qk, v = host(got["qk"]), host(got["v"])
    _, idx_o, margin_o, _ = orc.route(qk, mu0, sc.w)
    gidx = host(got["idx"])
    differs = check_membership(orc, gidx, idx_o, margin_o, qk, mu0, sc.w)
    o_r, _, _ = orc.routed_attn(qk, qk, v, gidx, scale, True)
    assert_rows_close(host(got["o_r"]), o_r, "routed heads")
    mu_o = orc.centroid_update(mu0, qk, qk, gidx, sc.lam)
    assert np.abs(host(got["mu"]) - mu_o).max() <= MU_MAX_ABS
    o_l = None
    if sc.L > 0:
        o_l = orc.local_attn(host(got["q_l"]), host(got["k_l"]), host(got["v_l"]), sc.window,
                             scale, True)
        assert_rows_close(host(got["o_l"]), o_l, "local heads")
    args_o = (host(got["o_r"]), None if sc.L == 0 else host(got["o_l"]), w_o, x_in)
    assert_bf16_rounding_close(host(got["y"]), orc.out_proj(*args_o), "layer output",
                               out_bound(orc, *args_o))
    return int(differs.sum())


SMALL_STACK = S.StackConfig(62, "small_stack", 1, 512, 256, 64, 2, 2, 8, 64, 64, 2)


@pytest.mark.parametrize("sc", [SMALL_STACK, SMALL_STACK.scaled(cfg_id=63, B=2, n=300, L=0, w=40),
                                SMALL_STACK.scaled(cfg_id=64, d=128, dm=384, R=1, L=1, k=4, w=128)],
                         ids=["small", "b2_no_local", "d128"])
def test_layer_small(rt, orc, sc):
    say(f"[case] layer {sc}")
    x = S.stack_x(sc)
    lw = S.stack_layer(sc, 0)
    scale = 1.0 / math.sqrt(sc.d)
    got = gpu_layer(rt, dev_tensor(x), {k_: dev_tensor(v_) for k_, v_ in lw.items()}, sc, scale)
    torch.cuda.synchronize()
    want = orc.layer_forward(x.value, lw["w_in"].value, lw["w_o"].value, lw["mu"], sc.R, sc.L,
                             sc.d, sc.w, sc.window, sc.lam)
    ndiff, kept = check_layer(orc, got, want, sc, x.value, lw["w_in"].value)
    say(f"[layer] {ndiff} clusters differ, {kept:.1%} of tokens compared")


def test_layer_full_size(rt, orc):
    """Layer 0 of the long stack at full size against the oracle's layer."""
    sc = S.STACKS["long_stack"]
    x = S.stack_x(sc)
    lw = S.stack_layer(sc, 0)
    scale = 1.0 / math.sqrt(sc.d)
    got = gpu_layer(rt, dev_tensor(x), {k_: dev_tensor(v_) for k_, v_ in lw.items()}, sc, scale)
    torch.cuda.synchronize()
    want = orc.layer_forward(x.value, lw["w_in"].value, lw["w_o"].value, lw["mu"], sc.R, sc.L,
                             sc.d, sc.w, sc.window, sc.lam)
    ndiff, kept = check_layer(orc, got, want, sc, x.value, lw["w_in"].value)
    say(f"[layer full] {ndiff} clusters differ, {kept:.1%} of tokens compared")
    assert kept > 0.5


SAMPLED_LAYERS = (1, 11, 21)


def test_stack_22_layers(rt, orc):
    """The 22-layer long stack runs end to end, stays finite and repeats
    bit-identically; layers 1, 11 and 21 are each checked stage by stage
    against the oracle on the device's own inputs (the residual stream grows
    with depth, so the layer output can cancel to far below its terms: it is
    held to the rounding rule of its own product instead of a relative
    tolerance)."""
    sc = S.STACKS["long_stack"]
    scale = 1.0 / math.sqrt(sc.d)
    host_layers = [S.stack_layer(sc, l) for l in range(sc.layers)]
    layers = [{k_: dev_tensor(v_) for k_, v_ in hl.items()} for hl in host_layers]
    outs = []
    sampled = {}
    for rep in range(2):
        x = dev_tensor(S.stack_x(sc))
        for l in range(sc.layers):
            if rep == 0 and l in SAMPLED_LAYERS:
                x_in = host(x)
            res = gpu_layer(rt, x, layers[l], sc, scale)
            if rep == 0 and l in SAMPLED_LAYERS:
                torch.cuda.synchronize()
                sampled[l] = (x_in, {k_: v_.clone() for k_, v_ in res.items()})
            x = res["y"]
        torch.cuda.synchronize()
        outs.append(x)
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1])
    for l, (x_in, got) in sampled.items():
        ndiff = check_layer_staged(orc, got, x_in, host_layers[l], sc, scale)
        say(f"[stack layer {l}] every stage matches the oracle on its own input; "
            f"{ndiff} clusters differ at a near-tie; max |x| {np.abs(x_in).max():.3g}")
