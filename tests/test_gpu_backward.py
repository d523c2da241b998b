"""GPU parity of the in-cluster attention backward (rt_routed_attn_bwd) against
the fp64 oracle, on the same seeded inputs and the oracle's membership.

Tolerance: the forward's rule scaled by the gradient's magnitude, i.e.
max-abs <= tol * max(1, max|oracle|) with tol = 1e-4 (float32 inputs) or
2e-2 (bfloat16 inputs, where P and dl are also rounded to bf16 for the matrix
products), plus mean-rel <= 5e-3 for bfloat16.
"""
import math
import sys

import numpy as np
import pytest
import torch

import synthetic as S
from _util import BF16_MAX_ABS, BF16_MEAN_REL, F32_MAX_ABS, dev_tensor, host

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
    return S.Config(cfg_id=kw.pop("cfg_id"), name=kw.pop("name", "bwd"), backward=True, **kw)


BWD = {
    "tiny_f32": S.CONFIGS["tiny"].scaled(backward=True),
    "ragged_d64": base(cfg_id=40, dtype="bf16", B=2, R=2, L=0, n=300, d=64, k=8, w=40, window=0),
    "d128": base(cfg_id=41, dtype="bf16", B=1, R=1, L=0, n=400, d=128, k=4, w=100, window=0),
    "d32": base(cfg_id=42, dtype="bf16", B=1, R=2, L=0, n=200, d=32, k=6, w=33, window=0),
    "d16": base(cfg_id=43, dtype="bf16", B=1, R=1, L=0, n=129, d=16, k=5, w=20, window=0),
    "w256_d64": base(cfg_id=44, dtype="bf16", B=1, R=1, L=0, n=1000, d=64, k=6, w=256,
                     window=0),
    "w128_d128": base(cfg_id=45, dtype="bf16", B=1, R=1, L=0, n=700, d=128, k=7, w=128,
                      window=0),
    # every token in all 8 clusters: ranks beyond the token slots overflow
    "all_clusters": base(cfg_id=46, dtype="bf16", B=1, R=1, L=0, n=100, d=64, k=8, w=100,
                         window=0),
    "d128_w64": base(cfg_id=50, dtype="bf16", B=1, R=2, L=0, n=300, d=128, k=5, w=64,
                     window=0),
    "w1": base(cfg_id=47, dtype="bf16", B=1, R=1, L=0, n=64, d=64, k=10, w=1, window=0),
    "w128_d64": base(cfg_id=51, dtype="bf16", B=1, R=1, L=0, n=500, d=64, k=6, w=128,
                     window=0),
    "f32_d64": base(cfg_id=48, dtype="f32", B=1, R=2, L=0, n=200, d=64, k=5, w=64, window=0),
    "skewed": base(cfg_id=49, dtype="bf16", B=1, R=2, L=0, n=2048, d=64, k=16, w=128,
                   window=0, skew=True),
}


def dout_for(cfg):
    return S.normal_tensor(1000 * cfg.cfg_id + S.TENSOR_IDS["dout"], (cfg.B, cfg.R, cfg.n, cfg.d),
                           cfg.dtype)


def assert_grad_close(got, want, dtype, what):
    err = np.abs(got - want)
    if err.size == 0:
        return
    mag = max(1.0, float(np.abs(want).max()))
    tol = (F32_MAX_ABS if dtype == "f32" else BF16_MAX_ABS) * mag
    at = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol, (f"{what}: max-abs {err.max():.3e} > {tol:.3e} at {at}: "
                              f"got {got[at]:.6g} want {want[at]:.6g}")
    if dtype != "f32":
        mean_rel = err.sum() / max(np.abs(want).sum(), 1e-30)
        assert mean_rel <= BF16_MEAN_REL, f"{what}: mean-rel {mean_rel:.3e} > {BF16_MEAN_REL}"


def run_bwd_case(rt, orc, cfg, causal=True, scale=None, distinct=False, heads=None):
    say(f"[case] bwd {cfg} causal={causal} scale={scale} distinct={distinct}")
    inp = S.make_inputs(cfg)
    dout = dout_for(cfg)
    sc = 1.0 / math.sqrt(cfg.d) if scale is None else scale
    q = dev_tensor(inp["qk"])
    v = dev_tensor(inp["v"])
    mu = dev_tensor(inp["mu"])
    g = dev_tensor(dout)
    q_val, v_val, g_val = inp["qk"].value, inp["v"].value, dout.value
    if distinct:
        kin = S.normal_tensor(1000 * cfg.cfg_id + 99, q_val.shape, cfg.dtype)
        kk, k_val = dev_tensor(kin), kin.value
    else:
        kk, k_val = q, q_val
    _, idx_o, _, _ = orc.route(q_val, inp["mu"], cfg.w)
    idx = torch.from_numpy(idx_o).cuda()
    q_inv, _ = rt.route(q, mu, cfg.w)
    k_inv = rt.route(kk, mu, cfg.w)[0] if distinct else q_inv
    _, lse = rt.routed_attn(q, kk, v, idx, q_inv, k_inv, scale=sc, causal=causal, want_lse=True,
                            out_dtype=torch.float32)
    dq, dk, dv = rt.routed_attn_bwd(q, kk, v, idx, lse, g, q_inv, k_inv, scale=sc, causal=causal)
    # again, with the membership bits given (built here from idx, as rt_route
    # writes them) instead of built by the call: the same gradients, bit for bit
    B_, H_, k_, w_ = idx_o.shape
    bits = np.zeros((B_, H_, cfg.n, (k_ + 31) // 32), dtype=np.uint32)
    bb, hh, cc, _ = np.indices(idx_o.shape)
    np.bitwise_or.at(bits, (bb, hh, idx_o, cc // 32), (np.uint32(1) << (cc % 32).astype(np.uint32)))
    mask = torch.from_numpy(bits.view(np.int32)).cuda()
    dq2, dk2, dv2 = rt.routed_attn_bwd(q, kk, v, idx, lse, g, q_inv, k_inv, scale=sc,
                                       causal=causal, mask=mask)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), \
        "backward is not deterministic, or differs with the membership bits given"
    dqk = None
    if not distinct:
        # shared q/k: the summed gradient dq_hat + dk_hat straight from the call,
        # deterministic, with the same dv
        dqk, none_, dv3 = rt.routed_attn_bwd(q, kk, v, idx, lse, g, q_inv, k_inv, scale=sc,
                                             causal=causal, mask=mask, sum_qk=True)
        dqk2, _, _ = rt.routed_attn_bwd(q, kk, v, idx, lse, g, q_inv, k_inv, scale=sc,
                                        causal=causal, mask=mask, sum_qk=True)
        torch.cuda.synchronize()
        assert none_ is None and torch.equal(dqk, dqk2) and torch.equal(dv3, dv)
        # the same sum as the two gradients added (float32 rounding of the sum apart)
        sep = host(dq) + host(dk)
        assert np.abs(host(dqk) - sep).max() <= 1e-5 * max(1.0, np.abs(sep).max())
    hs = range(cfg.R) if heads is None else heads
    for h in hs:
        sl = (slice(None), slice(h, h + 1))
        dq_o, dk_o, dv_o = orc.routed_attn_bwd(q_val[sl], k_val[sl], v_val[sl], idx_o[sl],
                                               g_val[sl], sc, causal)
        assert_grad_close(host(dq)[sl], dq_o, cfg.dtype, f"dq_hat head {h}")
        assert_grad_close(host(dk)[sl], dk_o, cfg.dtype, f"dk_hat head {h}")
        assert_grad_close(host(dv)[sl], dv_o, cfg.dtype, f"dv head {h}")
        if dqk is not None:
            assert_grad_close(host(dqk)[sl], dq_o + dk_o, cfg.dtype, f"dq_hat + dk_hat head {h}")
    # tokens no cluster holds get exactly zero gradients
    cnt = np.zeros((cfg.B, cfg.R, cfg.n), np.int64)
    for b in range(cfg.B):
        for h in range(cfg.R):
            cnt[b, h] = np.bincount(idx_o[b, h].ravel(), minlength=cfg.n)
    for t in (dq, dk, dv) + (() if dqk is None else (dqk,)):
        assert np.all(host(t)[cnt == 0] == 0.0)
    return cnt


@pytest.mark.parametrize("name", list(BWD))
def test_bwd_small(rt, orc, name):
    cnt = run_bwd_case(rt, orc, BWD[name])
    if name == "all_clusters":
        assert cnt.min() == 8


@pytest.mark.parametrize("name", ["ragged_d64", "d32", "tiny_f32", "w128_d128"])
def test_bwd_noncausal(rt, orc, name):
    run_bwd_case(rt, orc, BWD[name], causal=False)


@pytest.mark.parametrize("name", ["ragged_d64", "d16", "f32_d64", "w256_d64"])
def test_bwd_scale_sqrt_d(rt, orc, name):
    cfg = BWD[name]
    run_bwd_case(rt, orc, cfg, scale=math.sqrt(cfg.d))


@pytest.mark.parametrize("name", ["ragged_d64", "f32_d64", "d128_w64", "w128_d64", "tiny_f32"])
def test_bwd_distinct_q_and_k(rt, orc, name):
    run_bwd_case(rt, orc, BWD[name], distinct=True)


def test_bwd_limits(rt):
    """Clusters beyond what the backward keeps on chip are refused, not run."""
    q = torch.zeros((1, 1, 600, 128), dtype=torch.bfloat16, device="cuda")
    idx = torch.arange(129, dtype=torch.int32, device="cuda").reshape(1, 1, 1, 129)
    lse = torch.zeros((1, 1, 1, 129), dtype=torch.float32, device="cuda")
    with pytest.raises(rt.RTError, match="RT_EUNSUPPORTED"):
        rt.routed_attn_bwd(q, q, q, idx, lse, q)


def test_bwd_full_size_stress(rt, orc):
    """The stress workload at full size (n=32768, 8 heads, k=128, w=256, skewed
    tokens) in one launch; two heads are checked against the oracle."""
    run_bwd_case(rt, orc, S.CONFIGS["stress"], heads=[0, 5])
