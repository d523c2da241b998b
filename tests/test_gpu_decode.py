"""GPU parity of incremental decode against the fp64 oracle on the same seeded
inputs: cluster caches filled from a prefill membership (the oracle's routing
of the first n tokens), then several routed steps; local rings filled from a
prefill, then several local steps.

Rules.  Cache rows are bf16 copies: bit-exact; inverse norms within 2e-6
relative.  A step's cluster is a nearest-centroid decision taken from float32
scores on the device and float64 ones in the oracle: where the oracle's gap
between the two best centroids is below 1e-5 either choice is valid, so a
(batch, head) whose choice differs there must have taken one of the centroids
within 1e-5 of the best, and the oracle's step is re-run with the device's
choice, so that its later steps and caches are still compared; elsewhere the
labels must be equal.  Outputs: float32 within 1e-4, bfloat16 within the
bf16 rule.
"""
import math
import sys

import numpy as np
import pytest
import torch

import synthetic as S
from _util import assert_close_out, dev_tensor, host

pytestmark = pytest.mark.gpu
TIE = 1e-5


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


def label_slack(orc, x, mu, label):
    """[B, H] how far below the best centroid score the centroid `label` scores,
    for rows x [B,H,d] (the oracle's float64 scores)."""
    xh, _ = orc.normalize(x[:, :, None, :])
    s = np.einsum("bhd,hkd->bhk", xh[:, :, 0], mu)
    got = np.take_along_axis(s, label[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    return s.max(axis=2) - got


def compare_cache(got, want, live, what):
    """Caches of the (batch, head) pairs in `live` [B, H] (bool) must agree."""
    ln = host(got["len"])
    np.testing.assert_array_equal(ln[live], want["len"][live], err_msg=f"{what}: len")
    B, H, k = ln.shape
    gk, gv, gi, gp = host(got["k"]), host(got["v"]), host(got["inv"]), host(got["pos"])
    for b in range(B):
        for h in range(H):
            if not live[b, h]:
                continue
            for c in range(k):
                m = int(ln[b, h, c])
                np.testing.assert_array_equal(gk[b, h, c, :m], want["k"][b, h, c, :m])
                np.testing.assert_array_equal(gv[b, h, c, :m], want["v"][b, h, c, :m])
                np.testing.assert_array_equal(gp[b, h, c, :m], want["pos"][b, h, c, :m])
                np.testing.assert_allclose(gi[b, h, c, :m], want["inv"][b, h, c, :m], rtol=2e-6)


ROUTED = {
    # name: (B, H, n, d, k, w, slack, steps, out dtype)
    "d64_k8": (2, 2, 256, 64, 8, 32, 16, 12, torch.float32),
    "d128_k16_bf16out": (1, 4, 512, 128, 16, 32, 24, 16, torch.bfloat16),
    "d16_k1": (1, 2, 300, 16, 1, 300, 8, 5, torch.float32),     # one cluster: causal attention
    "d32_long_rows": (1, 2, 700, 32, 2, 350, 8, 6, torch.float32),  # > 256 entries a cluster
    "d64_k256": (1, 1, 512, 64, 256, 2, 12, 10, torch.float32),
}


def run_routed(rt, orc, B, H, n, d, k, w, slack, steps, odt, seed):
    tot = n + steps
    qk = S.normal_tensor(seed, (B, H, tot, d), "bf16")
    v = S.normal_tensor(seed + 1, (B, H, tot, d), "bf16")
    mu = S.unit_rows_f32(seed + 2, H * k, d).reshape(H, k, d)
    sc = 1.0 / math.sqrt(d)
    qk_pre, v_pre = qk.value[:, :, :n], v.value[:, :, :n]
    _, idx, _, _ = orc.route(qk_pre, mu, w)
    want = orc.decode_cache_from_prefill(qk_pre, v_pre, idx, w + slack)
    qk_d, v_d = dev_tensor(qk), dev_tensor(v)
    mu_d = torch.from_numpy(mu.astype(np.float32)).cuda()
    pre_qk, pre_v = qk_d[:, :, :n].contiguous(), v_d[:, :, :n].contiguous()
    inv_d, _ = rt.route(pre_qk, mu_d, w)
    cache = rt.decode_fill(pre_qk, pre_v, inv_d, torch.from_numpy(idx).cuda(), w + slack)
    torch.cuda.synchronize()
    live = np.ones((B, H), bool)
    compare_cache(cache, want, live, "fill")
    resynced = 0
    for t in range(n, tot):
        qk_t, v_t = qk_d[:, :, t].contiguous(), v_d[:, :, t].contiguous()
        out, label = rt.decode_routed(cache, qk_t, v_t, t, mu_d, scale=sc, out_dtype=odt)
        torch.cuda.synchronize()
        glab = host(label)
        prev = want
        wout, wlab, want = orc.decode_step(prev, qk.value[:, :, t], v.value[:, :, t], t, mu, sc)
        differ = glab != wlab
        if differ.any():
            slack = label_slack(orc, qk.value[:, :, t], mu, glab)
            assert np.all(slack[differ] < TIE), f"step {t}: labels differ away from a near-tie"
            # the device's choice is valid: the oracle takes it too and goes on
            wout, wlab, want = orc.decode_step(prev, qk.value[:, :, t], v.value[:, :, t], t, mu,
                                               sc, label_given=glab)
            resynced += int(differ.sum())
        got = host(out)
        assert_close_out(got, wout, "f32" if odt == torch.float32 else "bf16", f"step {t} out")
    compare_cache(cache, want, live, "after steps")
    return resynced


@pytest.mark.parametrize("name", list(ROUTED))
def test_decode_routed(rt, orc, name):
    say(f"[case] decode routed {name}")
    seed = 90_000 + 10 * list(ROUTED).index(name)
    resynced = run_routed(rt, orc, *ROUTED[name], seed)
    say(f"[decode routed] {resynced} steps took the other side of a near-tie (oracle re-synced)")


def test_decode_routed_full_size(rt, orc):
    """The long workload's routed heads (8 heads, n = 8192, d = 128, k = 64,
    w = 128): prefill caches, then 6 steps."""
    cfg = S.CONFIGS["long"]
    say("[case] decode routed long")
    resynced = run_routed(rt, orc, cfg.B, cfg.R, cfg.n, cfg.d, cfg.k, cfg.w, 32, 6,
                          torch.float32, 90_900)
    say(f"[decode routed long] {resynced} re-synced at a near-tie")


def test_decode_routed_full_cluster(rt, orc):
    """A cluster with no room left: label -1, NaN output row, caches unchanged
    for that (batch, head); the other heads step normally."""
    B, H, n, d, k, w = 1, 2, 64, 16, 1, 64
    qk = S.normal_tensor(90_950, (B, H, n + 1, d), "bf16")
    v = S.normal_tensor(90_951, (B, H, n + 1, d), "bf16")
    mu = S.unit_rows_f32(90_952, H * k, d).reshape(H, k, d)
    _, idx, _, _ = orc.route(qk.value[:, :, :n], mu, w)
    qk_d, v_d = dev_tensor(qk), dev_tensor(v)
    mu_d = torch.from_numpy(mu.astype(np.float32)).cuda()
    pre_qk, pre_v = qk_d[:, :, :n].contiguous(), v_d[:, :, :n].contiguous()
    inv_d, _ = rt.route(pre_qk, mu_d, w)
    cache = rt.decode_fill(pre_qk, pre_v, inv_d, torch.from_numpy(idx).cuda(), w)   # full
    cache["len"][0, 1] = w - 1                  # head 1 has room for one more entry
    before = {name: t.clone() for name, t in cache.items()}
    out, label = rt.decode_routed(cache, qk_d[:, :, n].contiguous(), v_d[:, :, n].contiguous(), n,
                                  mu_d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert host(label)[0, 0] == -1 and host(label)[0, 1] == 0
    assert np.all(np.isnan(host(out)[0, 0])) and np.all(np.isfinite(host(out)[0, 1]))
    for name in before:
        assert torch.equal(cache[name][0, 0], before[name][0, 0]), name
    assert int(cache["len"][0, 1, 0]) == w


LOCAL = {
    # name: (B, H, n, d, window, steps, out dtype)
    "d64_w32": (2, 2, 100, 64, 32, 40, torch.float32),
    "d128_w512_bf16out": (1, 2, 600, 128, 512, 8, torch.bfloat16),
    "short_prefill": (1, 1, 5, 32, 64, 70, torch.float32),    # ring not yet full, then wraps
    "d16_w1": (1, 2, 10, 16, 1, 3, torch.float32),
}


def run_local(rt, orc, B, H, n, d, window, steps, odt, seed):
    tot = n + steps
    q, kk, v = (S.normal_tensor(seed + i, (B, H, tot, d), "bf16") for i in range(3))
    sc = 1.0 / math.sqrt(d)
    wk = np.zeros((B, H, window, d))
    wv = np.zeros((B, H, window, d))
    for p in range(max(0, n - window), n):
        wk[:, :, p % window] = kk.value[:, :, p]
        wv[:, :, p % window] = v.value[:, :, p]
    q_d, k_d, v_d = dev_tensor(q), dev_tensor(kk), dev_tensor(v)
    rk, rv = rt.decode_ring_fill(k_d[:, :, :n].contiguous(), v_d[:, :, :n].contiguous(), window)
    torch.cuda.synchronize()
    filled = sorted({p % window for p in range(max(0, n - window), n)})
    np.testing.assert_array_equal(host(rk)[:, :, filled], wk[:, :, filled])
    np.testing.assert_array_equal(host(rv)[:, :, filled], wv[:, :, filled])
    for t in range(n, tot):
        out = rt.decode_local(rk, rv, q_d[:, :, t].contiguous(), k_d[:, :, t].contiguous(),
                              v_d[:, :, t].contiguous(), t, scale=sc, out_dtype=odt)
        torch.cuda.synchronize()
        want, wk, wv = orc.local_decode_step(wk, wv, q.value[:, :, t], kk.value[:, :, t],
                                             v.value[:, :, t], t, window, sc)
        assert_close_out(host(out), want, "f32" if odt == torch.float32 else "bf16",
                         f"step {t} out")
    np.testing.assert_array_equal(host(rk), wk)


@pytest.mark.parametrize("name", list(LOCAL))
def test_decode_local(rt, orc, name):
    say(f"[case] decode local {name}")
    run_local(rt, orc, *LOCAL[name], 91_000 + 10 * list(LOCAL).index(name))


def test_decode_local_from_start(rt, orc):
    """Steps from position 0 on zeroed rings (no prefill)."""
    B, H, d, window, steps = 1, 2, 64, 16, 24
    q, kk, v = (S.normal_tensor(91_500 + i, (B, H, steps, d), "bf16") for i in range(3))
    sc = 1.0 / math.sqrt(d)
    rk = torch.zeros((B, H, window, d), dtype=torch.bfloat16, device="cuda")
    rv = torch.zeros_like(rk)
    wk, wv = np.zeros((B, H, window, d)), np.zeros((B, H, window, d))
    q_d, k_d, v_d = dev_tensor(q), dev_tensor(kk), dev_tensor(v)
    for t in range(steps):
        out = rt.decode_local(rk, rv, q_d[:, :, t].contiguous(), k_d[:, :, t].contiguous(),
                              v_d[:, :, t].contiguous(), t, scale=sc, out_dtype=torch.float32)
        torch.cuda.synchronize()
        want, wk, wv = orc.local_decode_step(wk, wv, q.value[:, :, t], kk.value[:, :, t],
                                             v.value[:, :, t], t, window, sc)
        assert_close_out(host(out), want, "f32", f"step {t} out")


def test_decode_local_full_size(rt, orc):
    """The long workload's local heads (4 heads, n = 8192, d = 128, window 512)."""
    cfg = S.CONFIGS["long"]
    say("[case] decode local long")
    run_local(rt, orc, cfg.B, cfg.L, cfg.n, cfg.d, cfg.window, 6, torch.float32, 91_900)


def test_decode_local_matches_prefill_attention(rt, orc):
    """Position t's local decode output equals sliding-window attention over
    the whole sequence at position t (the oracle's prefill form)."""
    B, H, n, d, window, steps = 1, 2, 200, 64, 48, 5
    q, kk, v = (S.normal_tensor(91_700 + i, (B, H, n + steps, d), "bf16") for i in range(3))
    sc = 1.0 / math.sqrt(d)
    full = orc.local_attn(q.value, kk.value, v.value, window, sc)
    q_d, k_d, v_d = dev_tensor(q), dev_tensor(kk), dev_tensor(v)
    rk, rv = rt.decode_ring_fill(k_d[:, :, :n].contiguous(), v_d[:, :, :n].contiguous(), window)
    for t in range(n, n + steps):
        out = rt.decode_local(rk, rv, q_d[:, :, t].contiguous(), k_d[:, :, t].contiguous(),
                              v_d[:, :, t].contiguous(), t, scale=sc, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close_out(host(out), full[:, :, t], "f32", f"step {t}")
