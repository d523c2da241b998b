"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, on the
same seeded inputs.

Rules (see tests/_util.py): memberships equal wherever the oracle's top-w
score margin exceeds 1e-5 and valid elsewhere; attention outputs within
max-abs 1e-4 (float32) or max-abs 2e-2 and mean-rel 5e-3 (bfloat16);
centroids within max-abs 1e-5.  Outputs that depend on the membership are
compared twice: once with the oracle's membership fed to the GPU kernels,
once end to end on the tokens whose clusters the two sides chose alike.
"""
import math
import sys

import numpy as np
import pytest
import torch

import synthetic as S
from _util import (MU_MAX_ABS, assert_close_out, assert_exact_rounding, assert_mask_matches,
                   check_membership, dev_tensor, host, tokens_touched)

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


def base(**kw):
    return S.Config(cfg_id=kw.pop("cfg_id", 11), name=kw.pop("name", "case"), **kw)


# Small cases: several tiles, ragged tails, every supported d, edge shapes.
SMALL = {
    "tiny_f32": S.CONFIGS["tiny"],
    "tiny_bf16": S.CONFIGS["tiny"].scaled(dtype="bf16", cfg_id=12),
    "ragged_d64": base(cfg_id=13, dtype="bf16", B=2, R=2, L=2, n=1000, d=64, k=32, w=31,
                       window=100),
    "ragged_d128": base(cfg_id=14, dtype="bf16", B=1, R=2, L=1, n=777, d=128, k=6, w=100,
                        window=129),
    "d32": base(cfg_id=15, dtype="bf16", B=1, R=3, L=1, n=300, d=32, k=10, w=30, window=33),
    "d16": base(cfg_id=16, dtype="bf16", B=2, R=1, L=1, n=257, d=16, k=17, w=15, window=64),
    "dense_k1": base(cfg_id=17, dtype="bf16", B=1, R=2, L=0, n=200, d=64, k=1, w=200, window=0),
    "w1": base(cfg_id=18, dtype="bf16", B=1, R=1, L=0, n=130, d=64, k=40, w=1, window=0),
    "w_eq_n": base(cfg_id=19, dtype="bf16", B=1, R=1, L=0, n=128, d=32, k=3, w=128, window=0),
    "w256_d64": base(cfg_id=20, dtype="bf16", B=1, R=1, L=1, n=1500, d=64, k=5, w=256, window=256),
    "w512_d32": base(cfg_id=21, dtype="bf16", B=1, R=1, L=0, n=2000, d=32, k=3, w=512, window=0),
    "w256_d128": base(cfg_id=22, dtype="bf16", B=1, R=1, L=0, n=1100, d=128, k=4, w=256, window=0),
    "f32_d64": base(cfg_id=23, dtype="f32", B=1, R=2, L=1, n=333, d=64, k=5, w=40, window=50),
    "f32_d128": base(cfg_id=24, dtype="f32", B=1, R=1, L=1, n=200, d=128, k=3, w=64, window=70),
    "k_many": base(cfg_id=25, dtype="bf16", B=1, R=1, L=0, n=4096, d=64, k=256, w=16, window=0),
    "skewed": base(cfg_id=26, dtype="bf16", B=1, R=2, L=0, n=2048, d=64, k=16, w=128, window=0,
                   skew=True),
}


def run_routed_case(rt, orc, cfg, scale=None, causal=True, check_scores=True):
    say(f"[case] {cfg}")
    inp = S.make_inputs(cfg)
    sc = 1.0 / math.sqrt(cfg.d) if scale is None else scale
    qk = dev_tensor(inp["qk"])
    v = dev_tensor(inp["v"])
    mu = dev_tensor(inp["mu"])
    qk_val, v_val, mu_val = inp["qk"].value, inp["v"].value, inp["mu"]

    # route
    inv, idx, scores = rt.route(qk, mu, cfg.w, want_scores=True)
    torch.cuda.synchronize()
    inv_o, idx_o, margin_o, scores_o = orc.route(qk_val, mu_val, cfg.w, want_scores=check_scores)
    np.testing.assert_allclose(host(inv), inv_o, rtol=2e-6)
    if check_scores:
        err = np.abs(host(scores) - scores_o).max()
        assert err <= 2e-6, f"scores max-abs {err:.3e}"
    gidx = host(idx)
    differs = check_membership(orc, gidx, idx_o, margin_o, qk_val, mu_val, cfg.w)

    # attention with the oracle's membership (float32 output checked against
    # the tolerance; the storage-dtype output must be its exact rounding)
    idx_o_dev = torch.from_numpy(idx_o).cuda()
    out, lse = rt.routed_attn(qk, qk, v, idx_o_dev, inv, inv, scale=sc, causal=causal,
                              want_lse=True, out_dtype=torch.float32)
    out_st = rt.routed_attn(qk, qk, v, idx_o_dev, inv, inv, scale=sc, causal=causal)
    torch.cuda.synchronize()
    assert_exact_rounding(out_st, out)
    out_o, lse_o, _ = orc.routed_attn(qk_val, qk_val, v_val, idx_o, sc, causal)
    assert_close_out(host(out), out_o, cfg.dtype, "out")
    lse_tol = 1e-4 if cfg.dtype == "f32" else 5e-3
    assert np.abs(host(lse) - lse_o).max() <= lse_tol

    # centroid update with the oracle's membership
    mu2 = mu.clone()
    rt.centroid_update_(mu2, qk, inv, idx_o_dev, cfg.lam)
    torch.cuda.synchronize()
    mu_o = orc.centroid_update(mu_val, qk_val, qk_val, idx_o, cfg.lam)
    assert np.abs(host(mu2) - mu_o).max() <= MU_MAX_ABS

    # end to end on the GPU's own membership
    out_e = rt.routed_attn(qk, qk, v, idx, inv, inv, scale=sc, causal=causal,
                           out_dtype=torch.float32)
    mu_e = mu.clone()
    rt.centroid_update_(mu_e, qk, inv, idx, cfg.lam)
    torch.cuda.synchronize()
    keep = ~tokens_touched(gidx, idx_o, differs, cfg.n)
    assert_close_out(host(out_e)[keep], out_o[keep], cfg.dtype, "out end-to-end")
    same_c = ~differs.any(axis=0)                      # [H, k]: identical for every batch row
    assert np.abs(host(mu_e)[same_c] - mu_o[same_c]).max(initial=0.0) <= MU_MAX_ABS

    # fused path: membership bits from route, member sums from the attention
    inv_f, idx_f, mask_f = rt.route(qk, mu, cfg.w, want_mask=True)
    sum_q = torch.empty((cfg.B, cfg.R, cfg.k, cfg.d), dtype=torch.float32, device="cuda")
    out_f = rt.routed_attn(qk, qk, v, idx_f, inv_f, inv_f, scale=sc, causal=causal,
                           out_dtype=torch.float32, mask=mask_f, sums=(sum_q, None))
    mu_f = mu.clone()
    rt.centroid_update_sums_(mu_f, sum_q, cfg.lam)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx) and torch.equal(out_f, out_e)
    assert_mask_matches(host(mask_f), gidx, cfg.n)
    assert np.abs(host(mu_f)[same_c] - mu_o[same_c]).max(initial=0.0) <= MU_MAX_ABS

    # attention and update in one call: the same output and centroids, bit for bit
    mu_u = mu.clone()
    out_u = rt.routed_attn_update_(qk, qk, v, idx_f, inv_f, inv_f, mu_u, cfg.lam, scale=sc,
                                   causal=causal, out_dtype=torch.float32, mask=mask_f)
    torch.cuda.synchronize()
    assert torch.equal(out_u, out_f) and torch.equal(mu_u, mu_f)
    return dict(inp=inp, qk=qk, v=v, mu=mu, inv=inv, idx=idx, out=out_e, mu_e=mu_e, sc=sc,
                differs=differs)


@pytest.mark.parametrize("name", list(SMALL))
def test_routed_small(rt, orc, name):
    run_routed_case(rt, orc, SMALL[name])


@pytest.mark.parametrize("name", ["ragged_d64", "d32", "tiny_f32"])
def test_routed_noncausal(rt, orc, name):
    run_routed_case(rt, orc, SMALL[name], causal=False, check_scores=False)


@pytest.mark.parametrize("name", ["ragged_d128", "d16", "f32_d64", "w256_d64"])
def test_routed_scale_sqrt_d(rt, orc, name):
    cfg = SMALL[name]
    run_routed_case(rt, orc, cfg, scale=math.sqrt(cfg.d), check_scores=False)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_distinct_q_and_k(rt, orc, dtype):
    """Queries and keys from different tensors (each normalised by its own
    norm) with one membership (the oracle's routing of the queries); the key
    side of the EMA comes from the key tensor."""
    cfg = base(cfg_id=30, dtype=dtype, B=2, R=2, L=0, n=600, d=64, k=8, w=70, window=0)
    say(f"[case] distinct q/k {cfg}")
    inp = S.make_inputs(cfg)
    kin = S.normal_tensor(30_000 + 77, inp["qk"].value.shape, dtype)
    q, kk, v, mu = (dev_tensor(inp["qk"]), dev_tensor(kin), dev_tensor(inp["v"]),
                    dev_tensor(inp["mu"]))
    q_inv, idx = rt.route(q, mu, cfg.w)
    k_inv, _ = rt.route(kk, mu, cfg.w)
    _, idx_o, margin_o, _ = orc.route(inp["qk"].value, inp["mu"], cfg.w)
    check_membership(orc, host(idx), idx_o, margin_o, inp["qk"].value, inp["mu"], cfg.w)
    idx_o_dev = torch.from_numpy(idx_o).cuda()
    sc = 0.9
    sq = torch.empty((cfg.B, cfg.R, cfg.k, cfg.d), dtype=torch.float32, device="cuda")
    sk = torch.empty_like(sq)
    out = rt.routed_attn(q, kk, v, idx_o_dev, q_inv, k_inv, scale=sc, out_dtype=torch.float32,
                         sums=(sq, sk))
    out_st = rt.routed_attn(q, kk, v, idx_o_dev, q_inv, k_inv, scale=sc)
    assert_exact_rounding(out_st, out)
    mu2 = mu.clone()
    rt.centroid_update_(mu2, q, q_inv, idx_o_dev, 0.7, kk=kk, k_inv=k_inv)
    mu3 = mu.clone()
    rt.centroid_update_sums_(mu3, sq, 0.7, sum_k=sk)
    mu4 = mu.clone()
    out4 = rt.routed_attn_update_(q, kk, v, idx_o_dev, q_inv, k_inv, mu4, 0.7, scale=sc,
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out4, out) and torch.equal(mu4, mu3)
    out_o, _, _ = orc.routed_attn(inp["qk"].value, kin.value, inp["v"].value, idx_o, sc, True)
    assert_close_out(host(out), out_o, dtype)
    mu_o = orc.centroid_update(inp["mu"], inp["qk"].value, kin.value, idx_o, 0.7)
    assert np.abs(host(mu2) - mu_o).max() <= MU_MAX_ABS
    assert np.abs(host(mu3) - mu_o).max() <= MU_MAX_ABS


@pytest.mark.parametrize("lam", [0.0, 0.5, 1.0])
def test_centroid_update_lambdas(rt, orc, lam):
    cfg = SMALL["ragged_d64"]
    inp = S.make_inputs(cfg)
    qk, mu = dev_tensor(inp["qk"]), dev_tensor(inp["mu"])
    inv, idx = rt.route(qk, mu, cfg.w)
    _, idx_o, _, _ = orc.route(inp["qk"].value, inp["mu"], cfg.w)
    mu2 = mu.clone()
    rt.centroid_update_(mu2, qk, inv, torch.from_numpy(idx_o).cuda(), lam)
    torch.cuda.synchronize()
    mu_o = orc.centroid_update(inp["mu"], inp["qk"].value, inp["qk"].value, idx_o, lam)
    assert np.abs(host(mu2) - mu_o).max() <= MU_MAX_ABS
    if lam == 1.0:
        assert torch.equal(mu2, mu)


def test_unrouted_tokens_are_zero_and_deterministic(rt, orc):
    cfg = SMALL["ragged_d64"]
    res = run_routed_case(rt, orc, cfg, check_scores=False)
    idx = host(res["idx"])
    out = host(res["out"])
    for b in range(cfg.B):
        for h in range(cfg.R):
            cnt = np.bincount(idx[b, h].ravel(), minlength=cfg.n)
            assert np.all(out[b, h, cnt == 0] == 0.0)
            assert np.any(cnt == 0) and np.any(cnt >= 2)
    # bit-identical repeats
    qk, v, mu = res["qk"], res["v"], res["mu"]
    for _ in range(2):
        inv2, idx2 = rt.route(qk, mu, cfg.w)
        out2 = rt.routed_attn(qk, qk, v, idx2, inv2, inv2, scale=res["sc"],
                              out_dtype=torch.float32)
        mu3 = mu.clone()
        rt.centroid_update_(mu3, qk, inv2, idx2, cfg.lam)
        torch.cuda.synchronize()
        assert torch.equal(idx2, res["idx"]) and torch.equal(inv2, res["inv"])
        assert torch.equal(out2, res["out"]) and torch.equal(mu3, res["mu_e"])


@pytest.mark.parametrize("shape", [(2, 3, 300, 64, 10, 40, "bf16"), (1, 8, 8192, 128, 64, 128, "bf16"),
                                   (1, 2, 257, 32, 9, 33, "f32")],
                         ids=["ragged", "long", "f32"])
def test_two_stage_matches_routed_attn(rt, shape):
    """rt_cluster_attn then rt_scatter_rows (with and without the update) give
    rt_routed_attn's and rt_routed_attn_update's results bit for bit."""
    B, H, n, d, k, w, dtype = shape
    print(f"[case] two-stage {shape}", flush=True)
    qk = dev_tensor(S.normal_tensor(99_000, (B, H, n, d), dtype))
    v = dev_tensor(S.normal_tensor(99_001, (B, H, n, d), dtype))
    mu0 = torch.from_numpy(S.unit_rows_f32(99_002, H * k, d).reshape(H, k, d).astype(np.float32)).cuda()
    inv, idx, mask = rt.route(qk, mu0, w, want_mask=True)
    sc = 1.0 / math.sqrt(d)
    for odt in (torch.float32, qk.dtype):
        want, want_lse = rt.routed_attn(qk, qk, v, idx, inv, inv, scale=sc, mask=mask,
                                        want_lse=True, out_dtype=odt)
        mu_want = mu0.clone()
        want_u = rt.routed_attn_update_(qk, qk, v, idx, inv, inv, mu_want, 0.9, scale=sc,
                                        mask=mask, out_dtype=odt)
        sum_q = torch.empty((B, H, k, d), dtype=torch.float32, device="cuda")
        lse = torch.empty_like(want_lse)
        out, ws = rt.cluster_attn(qk, qk, v, idx, inv, inv, mask, scale=sc, out_dtype=odt,
                                  lse=lse, sums=(sum_q, None))
        rt.scatter_rows(mask, out, ws, k, w, in_dtype=qk.dtype)
        out2, ws2 = rt.cluster_attn(qk, qk, v, idx, inv, inv, mask, scale=sc, out_dtype=odt,
                                    sums=(sum_q, None))
        mu = mu0.clone()
        rt.scatter_rows(mask, out2, ws2, k, w, in_dtype=qk.dtype, mu=mu, sum_q=sum_q, lam=0.9)
        torch.cuda.synchronize()
        assert torch.equal(out, want) and torch.equal(lse, want_lse)
        assert torch.equal(out2, want_u) and torch.equal(mu, mu_want)


def test_binding_rejects_bad_shapes(rt):
    """The binding checks every buffer the kernels index by the shape
    arguments alone before anything is launched."""
    B, H, n, d, k, w = 1, 2, 128, 64, 8, 16
    qk = torch.randn((B, H, n, d), device="cuda").to(torch.bfloat16)
    v = torch.randn_like(qk)
    mu = torch.nn.functional.normalize(torch.randn((H, k, d), device="cuda"), dim=-1)
    inv, idx, mask = rt.route(qk, mu, w, want_mask=True)
    out, lse = rt.routed_attn(qk, qk, v, idx, inv, inv, mask=mask, want_lse=True)
    bad = {
        "mask": dict(mask=mask[:, :, : n - 1].contiguous()),
        "mask dtype": dict(mask=mask.to(torch.int64)),
        "lse": dict(lse=torch.empty((B, H, k, w - 1), device="cuda")),
        "q_inv": dict(q_inv=inv[:, :1].contiguous()),
    }
    for what, kw in bad.items():
        args = dict(q_inv=inv, k_inv=inv, mask=mask)
        args.update(kw)
        with pytest.raises(ValueError):
            rt.routed_attn(qk, qk, v, idx, args.pop("q_inv"), args.pop("k_inv"), **args)
    dout = torch.randn_like(qk)
    with pytest.raises(ValueError):
        rt.routed_attn_bwd(qk, qk, v, idx, lse[..., :-1].contiguous(), dout, inv, inv, mask=mask)
    with pytest.raises(ValueError):
        rt.routed_attn_bwd(qk, qk, v, idx, lse, dout[:, :1].contiguous(), inv, inv, mask=mask)
    with pytest.raises(ValueError):
        rt.routed_attn_update_(qk, qk, v, idx, inv, inv, mu[:, :-1].contiguous(), 0.9, mask=mask)
    torch.cuda.synchronize()


LOCAL = ["ragged_d64", "ragged_d128", "d32", "d16", "w256_d64", "f32_d64", "f32_d128"]


@pytest.mark.parametrize("name", LOCAL)
@pytest.mark.parametrize("causal", [True, False])
def test_local_small(rt, orc, name, causal):
    cfg = SMALL[name]
    say(f"[case] local {name} causal={causal}")
    inp = S.make_inputs(cfg)
    q, kk, v = (dev_tensor(inp[x]) for x in ("q_local", "k_local", "v_local"))
    sc = 1.0 / math.sqrt(cfg.d)
    out = rt.local_attn(q, kk, v, cfg.window, scale=sc, causal=causal, out_dtype=torch.float32)
    out_st = rt.local_attn(q, kk, v, cfg.window, scale=sc, causal=causal)
    torch.cuda.synchronize()
    assert_exact_rounding(out_st, out)
    out_o = orc.local_attn(inp["q_local"].value, inp["k_local"].value, inp["v_local"].value,
                           cfg.window, sc, causal)
    assert_close_out(host(out), out_o, cfg.dtype, "local out")


@pytest.mark.parametrize("window", [1, 7, 64, 5000])
def test_local_window_edges(rt, orc, window):
    cfg = SMALL["ragged_d64"]
    inp = S.make_inputs(cfg)
    q, kk, v = (dev_tensor(inp[x]) for x in ("q_local", "k_local", "v_local"))
    out = rt.local_attn(q, kk, v, window, scale=0.3, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out_o = orc.local_attn(inp["q_local"].value, inp["k_local"].value, inp["v_local"].value,
                           window, 0.3, True)
    assert_close_out(host(out), out_o, cfg.dtype, "local out")
    if window == 1:
        assert torch.equal(out, v.float())


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
@pytest.mark.parametrize("causal", [True, False])
def test_local_scale_signs(rt, orc, scale, causal):
    """Negative, zero and large scales (the kernel keeps its log2 scale positive
    by negating the queries, and treats zero as uniform weights)."""
    cfg = SMALL["ragged_d128"]
    inp = S.make_inputs(cfg)
    q, kk, v = (dev_tensor(inp[x]) for x in ("q_local", "k_local", "v_local"))
    out = rt.local_attn(q, kk, v, 50, scale=scale, causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out_o = orc.local_attn(inp["q_local"].value, inp["k_local"].value, inp["v_local"].value,
                           50, scale, causal)
    assert_close_out(host(out), out_o, cfg.dtype, "local out")


# The longest rows of the sequence-length sweep (k = sqrt(n)): the top-w variants
# for n = 16K (registers) and 64K (the 1024-thread register variant), 2 heads.
@pytest.mark.parametrize("n,k", [(16384, 128), (65536, 256)])
def test_sweep_long_rows(rt, orc, n, k):
    cfg = base(cfg_id=85 + (n == 65536), dtype="bf16", B=1, R=2, L=0, n=n, d=128, k=k, w=n // k,
               window=0)
    res = run_routed_case(rt, orc, cfg, check_scores=False)
    say(f"[sweep] n={n}: {int(res['differs'].sum())} near-tie clusters differ")


# Selection paths of the top-w kernel, for each place its keys live (full keys
# in registers up to n = 8K, their high halves beyond): exact ties
# (tokens drawn from a pool of 97 vectors), a threshold deep in a crowded top
# byte (tokens close to one direction: more candidates than the short list
# holds, even at 16-bit prefixes), a top byte too crowded for the short lists
# whose 16-bit prefixes are not (tokens spread about one direction, a centroid
# of norm 1.9 along it: scores 1.2 .. 1.5, all in the top byte [0.5, 2)), and a
# threshold below the four highest top bytes (w = n/2).
TOPW_PATHS = {"ties": (97, None), "crowded": (None, 0.01), "refine": (None, 1.0),
              "median": (None, None)}


def run_topw_case(rt, orc, n, kind, H, k, cid):
    """One route call on inputs built to take `kind`'s selection path, checked
    against the oracle: membership (margin rule), the bitmask, and for exact
    ties the lowest positions taken."""
    d = 64
    pool, spread = TOPW_PATHS[kind]
    if pool is not None:
        base_rows = S.normal(1000 * cid + 1, (pool, d))
        val = np.tile(base_rows[np.arange(n) % pool], (H, 1, 1))
    elif spread is not None:
        centre = S.normal(1000 * cid + 1, (1, d))
        val = centre + spread * S.normal(1000 * cid + 2, (H, n, d))
    else:
        val = S.normal(1000 * cid + 1, (H, n, d))
    qk_t = S.rounded(val.reshape(1, H, n, d), "bf16")
    mu_val = S.unit_rows_f32(1000 * cid + 3, H * k, d).reshape(H, k, d)
    if kind == "refine":
        unit = centre[0] / np.sqrt((centre[0] ** 2).sum())
        mu_val = mu_val.copy()
        mu_val[0, 0] = (1.9 * unit).astype(np.float32).astype(np.float64)
    w = n // 2 if kind == "median" else min(n // k, 1024)
    qk = dev_tensor(qk_t)
    mu = dev_tensor(mu_val)
    inv, idx, mask = rt.route(qk, mu, w, want_mask=True)
    torch.cuda.synchronize()
    _, idx_o, margin_o, _ = orc.route(qk_t.value, mu_val, w)
    gidx = host(idx)
    check_membership(orc, gidx, idx_o, margin_o, qk_t.value, mu_val, w)
    assert_mask_matches(host(mask), gidx, n)
    if kind == "ties":
        # equal scores are taken in position order: the chosen set is the
        # lowest positions among the tokens tied at the threshold
        xhat, _ = orc.normalize(qk_t.value[0, 0])
        for c in range(k):
            s = orc.scores(xhat, mu_val[0, c:c + 1])[0]
            row = gidx[0, 0, c]
            thr = s[row].min()
            tied = np.flatnonzero(s == thr)
            taken = np.intersect1d(row, tied)
            assert np.array_equal(taken, tied[:len(taken)])


@pytest.mark.parametrize("n", [3000, 20000, 40000, 65536])
@pytest.mark.parametrize("kind", list(TOPW_PATHS))
def test_topw_selection_paths(rt, orc, n, kind):
    say(f"[topw] n={n} kind={kind}")
    run_topw_case(rt, orc, n, kind, H=1, k=2, cid=88 + list(TOPW_PATHS).index(kind))


@pytest.mark.parametrize("n", [1024, 777])
@pytest.mark.parametrize("kind", list(TOPW_PATHS))
def test_topw_selection_paths_one_wave(rt, orc, n, kind):
    """The same paths where rows of up to 1024 keys, 1024 rows or more, take
    one wave a row (16 heads of 64 centroids)."""
    say(f"[topw one wave] n={n} kind={kind}")
    run_topw_case(rt, orc, n, kind, H=16, k=64, cid=92 + list(TOPW_PATHS).index(kind))


# Full-size workloads, in the launch configuration the benchmark times.
@pytest.mark.parametrize("name", ["routed", "mixed", "long", "stress"])
def test_full_size_forward(rt, orc, name):
    cfg = S.CONFIGS[name]
    res = run_routed_case(rt, orc, cfg, check_scores=False)
    say(f"[full] {name}: {int(res['differs'].sum())} near-tie clusters differ")
    if cfg.L > 0:
        inp = res["inp"]
        q, kk, v = (dev_tensor(inp[x]) for x in ("q_local", "k_local", "v_local"))
        out = rt.local_attn(q, kk, v, cfg.window, scale=res["sc"], out_dtype=torch.float32)
        torch.cuda.synchronize()
        out_o = orc.local_attn(inp["q_local"].value, inp["k_local"].value, inp["v_local"].value,
                               cfg.window, res["sc"], True)
        assert_close_out(host(out), out_o, cfg.dtype, "local out")
