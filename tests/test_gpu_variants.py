"""GPU parity of the variants (blocked local attention, the nearest-centroid
update, partition-style routing) against the fp64 oracle on the same seeded
inputs.

Rules.  Blocked local attention: as the local heads (float32 output within
1e-4 for float32 inputs; 2e-2 max-abs and 5e-3 mean-rel for bfloat16).  A
token's nearest centroid is a decision taken from float32-accurate scores on
the device and float64 ones in the oracle: where the oracle's gap between the
two best scores is below 1e-5 either choice is valid, so the centroids whose
members such a token could change are left out of the comparison; the others
within 1e-5.  Partition: every token in exactly one cluster of n/k, rows in
ascending position, and each token in a cluster its place in the oracle's
order (nearest centroid, descending score, position) allows, where keys
within 1e-5 of each other may be ordered either way; on inputs built free of
near-ties, every cluster equal to the oracle's.
Separately routed queries and keys: on the oracle's memberships, outputs as
the routed attention, log-sum-exp within 1e-4 (float32) / 5e-3 (bfloat16),
member sums within 1e-4 per 32 rows.
"""
import math
import sys

import numpy as np
import pytest
import torch

import synthetic as S
from _util import MU_MAX_ABS, assert_close_out, check_partition, dev_tensor, host

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


# ---- blocked local attention ------------------------------------------------------------

BLOCKED = {
    # name: (dtype, B, H, n, d, block, lookback)
    "d64_b50": ("bf16", 1, 2, 300, 64, 50, 1),
    "d128_b64": ("bf16", 2, 1, 257, 128, 64, 1),
    "own_block": ("bf16", 1, 1, 200, 64, 16, 0),
    "d32_b7_l2": ("bf16", 1, 1, 333, 32, 7, 2),
    "d128_b512": ("bf16", 1, 2, 1000, 128, 512, 1),
    "f32": ("f32", 1, 1, 130, 64, 20, 1),
}


@pytest.mark.parametrize("name", list(BLOCKED))
def test_local_attn_blocked(rt, orc, name):
    dtype, B, H, n, d, block, lookback = BLOCKED[name]
    say(f"[case] blocked {name}")
    seed = 80_000 + 10 * list(BLOCKED).index(name)
    q, kk, v = (S.normal_tensor(seed + i, (B, H, n, d), dtype) for i in range(3))
    sc = 1.0 / math.sqrt(d)
    out = rt.local_attn_blocked(dev_tensor(q), dev_tensor(kk), dev_tensor(v), block, lookback,
                                scale=sc, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = orc.local_attn_blocked(q.value, kk.value, v.value, block, lookback, sc)
    assert_close_out(host(out), want, dtype, "blocked out")


def test_local_attn_blocked_full_size(rt, orc):
    """The long workload's local heads as blocks of 512 with one block of look-back."""
    cfg = S.CONFIGS["long"]
    inp = S.make_inputs(cfg)
    sc = 1.0 / math.sqrt(cfg.d)
    out = rt.local_attn_blocked(dev_tensor(inp["q_local"]), dev_tensor(inp["k_local"]),
                                dev_tensor(inp["v_local"]), cfg.window, 1, scale=sc,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = orc.local_attn_blocked(inp["q_local"].value, inp["k_local"].value,
                                  inp["v_local"].value, cfg.window, 1, sc)
    assert_close_out(host(out), want, "bf16", "blocked out")


# ---- nearest-centroid update ------------------------------------------------------------

def fragile_centroids(orc, x, mu):
    """[H, k] mask of centroids whose member set a near-tie could change."""
    H, k = mu.shape[0], mu.shape[1]
    bad = np.zeros((H, k), bool)
    xh, _ = orc.normalize(x)
    B = x.shape[0]
    for b in range(B):
        for h in range(H):
            s = xh[b, h] @ mu[h].T                          # [n, k]
            srt = np.sort(s, axis=1)
            near = srt[:, -1] - srt[:, -2] < TIE if k > 1 else np.zeros(len(s), bool)
            for t in np.flatnonzero(near):
                bad[h, np.flatnonzero(s[t] >= srt[t, -1] - TIE)] = True
    return bad


EMA = {
    # name: (dtype, B, H, n, d, k, shared)
    "shared_bf16": ("bf16", 2, 2, 700, 64, 16, True),
    "distinct_bf16": ("bf16", 1, 2, 513, 128, 8, False),
    "f32_d32": ("f32", 2, 1, 300, 32, 5, True),
    "k1": ("bf16", 1, 1, 100, 64, 1, True),
    "long": ("bf16", 1, 8, 8192, 128, 64, True),
}


@pytest.mark.parametrize("name", list(EMA))
def test_centroid_update_argmax(rt, orc, name):
    dtype, B, H, n, d, k, shared = EMA[name]
    say(f"[case] argmax EMA {name}")
    seed = 81_000 + 10 * list(EMA).index(name)
    q = S.normal_tensor(seed, (B, H, n, d), dtype)
    kk = q if shared else S.normal_tensor(seed + 1, (B, H, n, d), dtype)
    mu0 = S.unit_rows_f32(seed + 2, H * k, d).reshape(H, k, d)
    mu = torch.from_numpy(mu0.astype(np.float32)).cuda()
    rt.centroid_update_argmax_(mu, dev_tensor(q), None if shared else dev_tensor(kk), lam=0.9)
    torch.cuda.synchronize()
    want = orc.centroid_update_argmax(mu0, q.value, kk.value, 0.9)
    skip = fragile_centroids(orc, q.value, mu0)
    if not shared:
        skip |= fragile_centroids(orc, kk.value, mu0)
    got = host(mu)
    assert (~skip).any()
    err = np.abs(got - want)[~skip]
    assert err.max() <= MU_MAX_ABS, f"max err {err.max():.3e}"
    say(f"[argmax EMA] {int(skip.sum())} of {skip.size} centroids near a tie")


def test_centroid_update_argmax_deterministic(rt):
    dtype, B, H, n, d, k, shared = EMA["shared_bf16"]
    q = dev_tensor(S.normal_tensor(81_900, (B, H, n, d), dtype))
    mu0 = torch.from_numpy(S.unit_rows_f32(81_901, H * k, d).reshape(H, k, d).astype(np.float32)).cuda()
    a, b = mu0.clone(), mu0.clone()
    rt.centroid_update_argmax_(a, q, lam=0.5)
    rt.centroid_update_argmax_(b, q, lam=0.5)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---- partition-style routing ------------------------------------------------------------

PART = {
    # name: (dtype, B, H, n, d, k)
    "bf16_d64": ("bf16", 2, 2, 512, 64, 8),
    "bf16_d128_k1": ("bf16", 1, 1, 256, 128, 1),
    "f32_d32": ("f32", 1, 2, 300, 32, 10),
    "k_eq_n": ("bf16", 1, 1, 64, 16, 64),
    "long": ("bf16", 1, 8, 8192, 128, 64),
    "n16k": ("bf16", 1, 8, 16384, 128, 128),
}


def run_partition(rt, orc, x, mu0, name):
    B, H, n, d = x.value.shape
    k = mu0.shape[1]
    inv, idx, mask = rt.route_partition(dev_tensor(x), torch.from_numpy(mu0.astype(np.float32)).cuda(),
                                        want_mask=True)
    torch.cuda.synchronize()
    _, want_inv = orc.normalize(x.value)
    np.testing.assert_allclose(host(inv), want_inv, rtol=2e-6)
    got = host(idx)
    m = host(mask).astype(np.int64) & 0xffffffff
    for b in range(B):
        for h in range(H):
            g = got[b, h]
            for c in range(k):                       # one bit per token, its cluster's
                assert np.all((m[b, h, g[c], c // 32] >> (c % 32)) & 1 == 1)
            assert int(sum(bin(int(x_)).count("1") for x_ in m[b, h].ravel())) == n
    pinned, free = check_partition(orc, got, x.value, mu0)
    say(f"[partition {name}] {pinned} tokens in the one cluster their rank allows, "
        f"{free} with a choice at a near-tie")
    return got, pinned, free


@pytest.mark.parametrize("name", list(PART))
def test_route_partition(rt, orc, name):
    """Every token sits in a cluster its oracle rank allows (near-ties widen
    the range only for the tokens they touch), on every (batch, head)."""
    dtype, B, H, n, d, k = PART[name]
    say(f"[case] partition {name}")
    seed = 82_000 + 10 * list(PART).index(name)
    x = S.normal_tensor(seed, (B, H, n, d), dtype)
    mu0 = S.unit_rows_f32(seed + 1, H * k, d).reshape(H, k, d)
    _, pinned, free = run_partition(rt, orc, x, mu0, name)
    assert pinned >= 0.95 * B * H * n


SEPARATED = {
    # name: (B, H, n, d, k)
    "long": (1, 8, 8192, 128, 64),
    "n16k": (1, 8, 16384, 128, 128),
    "d64_ragged_groups": (2, 2, 2048, 64, 16),
}


@pytest.mark.parametrize("name", list(SEPARATED))
def test_route_partition_separated_exact(rt, orc, name):
    """Tokens around separated centres with groups of unequal size (so the cuts
    fall inside groups and the score order decides them) and scores at least
    1e-3 apart: no near-tie exists, so every cluster of every (batch, head)
    must equal the oracle's."""
    B, H, n, d, k = SEPARATED[name]
    say(f"[case] partition separated {name}")
    x, mu0 = S.separated_tokens(97_000 + 10 * list(SEPARATED).index(name), B, H, n, d, k)
    got, pinned, free = run_partition(rt, orc, x, mu0, name)
    assert free == 0, "the input holds a near-tie"
    np.testing.assert_array_equal(got, orc.route_partition(x.value, mu0))


SKEWED = {
    # name: (B, H, n, d, k, weight of group 0 against 1 for the others)
    "one_large_group": (1, 2, 4096, 64, 16, 20.0),
    "nearly_all_one_group": (1, 1, 4096, 64, 16, 1000.0),
}


@pytest.mark.parametrize("name", list(SKEWED))
def test_route_partition_skewed_groups(rt, orc, name):
    """Most tokens nearest one centroid: that group holds thousands of members,
    so ranking them inside the group spans several tiles of members and several
    rounds of them per thread.  Every token must sit in a cluster its oracle
    rank allows, on every (batch, head)."""
    B, H, n, d, k, w0 = SKEWED[name]
    say(f"[case] partition skewed {name}")
    weights = np.ones(k)
    weights[0] = w0
    x, mu0 = S.separated_tokens(98_000 + 10 * list(SKEWED).index(name), B, H, n, d, k,
                                spacing=0.3 / n, weights=weights)
    got, pinned, free = run_partition(rt, orc, x, mu0, name)
    assert pinned >= 0.9 * B * H * n


def test_partition_clusters_feed_routed_attention(rt, orc):
    """Partition clusters are ordinary memberships: routed attention on the
    device's partition against the oracle's attention on the same partition."""
    dtype, B, H, n, d, k = PART["bf16_d64"]
    x = S.normal_tensor(82_500, (B, H, n, d), dtype)
    v = S.normal_tensor(82_501, (B, H, n, d), dtype)
    mu0 = S.unit_rows_f32(82_502, H * k, d).reshape(H, k, d)
    xd = dev_tensor(x)
    inv, idx = rt.route_partition(xd, torch.from_numpy(mu0.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    got_idx = host(idx)
    check_partition(orc, got_idx, x.value, mu0)
    sc = 1.0 / math.sqrt(d)
    out = rt.routed_attn(xd, xd, dev_tensor(v), idx, inv, inv, scale=sc, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want, _, _ = orc.routed_attn(x.value, x.value, v.value, got_idx, sc, True)
    assert_close_out(host(out), want, dtype, "routed out on partition clusters")


# ---- separately routed queries and keys ----------------------------------------------------

SPLIT = {
    # name: (dtype, B, H, n, d, k, w)
    "bf16_d64": ("bf16", 2, 2, 256, 64, 8, 32),
    "bf16_d128_w128": ("bf16", 1, 2, 1000, 128, 16, 128),
    "bf16_d32_ragged": ("bf16", 1, 1, 333, 32, 5, 70),
    "f32_d32": ("f32", 1, 2, 200, 32, 6, 40),
    "k1_w_eq_n": ("bf16", 1, 1, 96, 64, 1, 96),
}


def run_split(rt, orc, dtype, B, H, n, d, k, w, seed, want_sums=True):
    q = S.normal_tensor(seed, (B, H, n, d), dtype)
    kk = S.normal_tensor(seed + 1, (B, H, n, d), dtype)
    v = S.normal_tensor(seed + 2, (B, H, n, d), dtype)
    mu0 = S.unit_rows_f32(seed + 3, H * k, d).reshape(H, k, d)
    _, idx_q, _, _ = orc.route(q.value, mu0, w)
    _, idx_k, _, _ = orc.route(kk.value, mu0, w)
    mu = torch.from_numpy(mu0.astype(np.float32)).cuda()
    qd, kd, vd = dev_tensor(q), dev_tensor(kk), dev_tensor(v)
    q_inv, _ = rt.route(qd, mu, w)
    k_inv, _ = rt.route(kd, mu, w)
    iq, ik = torch.from_numpy(idx_q).cuda(), torch.from_numpy(idx_k).cuda()
    sc = 1.0 / math.sqrt(d)
    out, lse, sum_q, sum_k = rt.routed_attn_split(qd, kd, vd, iq, ik, q_inv, k_inv, scale=sc,
                                                  out_dtype=torch.float32, want_lse=True,
                                                  want_sums=True)
    torch.cuda.synchronize()
    want, want_lse, want_sq, want_sk = orc.routed_attn_split(q.value, kk.value, v.value, idx_q,
                                                             idx_k, sc)
    assert_close_out(host(out), want, dtype, "split out")
    # the bf16 kernels sum the bf16-rounded probabilities: the routed attention's rule
    assert np.abs(host(lse) - want_lse).max() <= (1e-4 if dtype == "f32" else 5e-3)
    np.testing.assert_allclose(host(sum_q), want_sq, atol=1e-4 * max(1, w / 32))
    np.testing.assert_allclose(host(sum_k), want_sk, atol=1e-4 * max(1, w / 32))
    return qd, kd, vd, iq, ik, q_inv, k_inv, out


@pytest.mark.parametrize("name", list(SPLIT))
def test_routed_attn_split(rt, orc, name):
    say(f"[case] split {name}")
    run_split(rt, orc, *SPLIT[name], 83_000 + 10 * list(SPLIT).index(name))


def test_routed_attn_split_one_membership_matches_noncausal(rt, orc):
    """With idx_q == idx_k the split entry point is rt_routed_attn without the
    causal mask, bit for bit."""
    dtype, B, H, n, d, k, w = SPLIT["bf16_d64"]
    qd, kd, vd, iq, ik, q_inv, k_inv, _ = run_split(rt, orc, dtype, B, H, n, d, k, w, 83_900)
    a = rt.routed_attn_split(qd, kd, vd, iq, iq, q_inv, k_inv, out_dtype=torch.float32)
    b = rt.routed_attn(qd, kd, vd, iq, q_inv, k_inv, causal=False, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_routed_attn_split_full_size(rt, orc):
    """The long workload's routed heads with distinct query and key vectors."""
    cfg = S.CONFIGS["long"]
    say("[case] split long")
    run_split(rt, orc, "bf16", cfg.B, cfg.R, cfg.n, cfg.d, cfg.k, cfg.w, 83_950)


# ---- Jensen-Shannon divergence between local and routed attention --------------------------

JS_TOL = 2e-3     # the local denominator is the local kernel's (bf16 probabilities, fp32 sum)

JS = {
    # name: (B, H, n, d, k, w, window, causal)
    "d64_w32": (1, 2, 300, 64, 6, 40, 32, True),
    "d128_w64": (1, 1, 1000, 128, 8, 128, 64, True),
    "d32_noncausal": (1, 2, 200, 32, 5, 50, 16, False),
    "d16_window1": (2, 1, 128, 16, 4, 32, 1, True),
}


def run_js(rt, orc, B, H, n, d, k, w, window, causal, seed, clusters=None):
    qk, ql, kl = (S.normal_tensor(seed + i, (B, H, n, d), "bf16") for i in range(3))
    mu0 = S.unit_rows_f32(seed + 3, H * k, d).reshape(H, k, d)
    _, idx, _, _ = orc.route(qk.value, mu0, w)
    qd = dev_tensor(qk)
    q_inv, _ = rt.route(qd, torch.from_numpy(mu0.astype(np.float32)).cuda(), w)
    sr, sl = 2.0, 1.0 / math.sqrt(d)
    js = rt.attn_js(qd, q_inv, torch.from_numpy(idx).cuda(), dev_tensor(ql), dev_tensor(kl), window,
                    scale_r=sr, scale_l=sl, causal=causal)
    torch.cuda.synchronize()
    got = host(js)
    assert np.all(got >= 0) and np.all(got <= math.log(2) + 1e-7)
    sel = list(range(k)) if clusters is None else clusters
    want = orc.attn_js(qk.value, idx[:, :, sel], ql.value, kl.value, window, sr, sl, causal)
    err = np.abs(got[:, :, sel] - want)
    assert err.max() <= JS_TOL, f"max err {err.max():.3e}"
    return got


@pytest.mark.parametrize("name", list(JS))
def test_attn_js(rt, orc, name):
    say(f"[case] js {name}")
    run_js(rt, orc, *JS[name], 84_000 + 10 * list(JS).index(name))


def test_attn_js_full_size(rt, orc):
    """The long workload's routed heads against a local head each (one batch
    row, 8 heads, n = 8192, k = 64, w = 128, window 512); the oracle on three
    clusters."""
    cfg = S.CONFIGS["long"]
    say("[case] js long")
    got = run_js(rt, orc, cfg.B, 2, cfg.n, cfg.d, cfg.k, cfg.w, cfg.window, True, 84_900,
                 clusters=[0, 31, 63])
    say(f"[js long] mean {got.mean():.4f}")
