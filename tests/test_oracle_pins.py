"""Pins of the fp64 CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a library routine for a
special case the method reduces to (torch's scaled_dot_product_attention and
autograd in float64, numpy sorting, scipy distances), brute force on tiny
inputs, or hand-derived values (tests/golden/hand_example.json).  The pages
describe the method in words (paperlayer.ai summary of "Efficient
Content-Based Sparse Attention with Routing Transformers", §3 attention, §4
routing attention with clustering and balanced clusters, §2/§4 online
spherical k-means centroids shared across sequences).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.spatial.distance import cdist

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")
TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(a):
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


def _sdpa(q, k, v, scale, causal=True, mask=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)
    return F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask,
                                          is_causal=causal and mask is None,
                                          scale=scale).numpy()


def _ev(expr):
    return eval(expr, {"ln2": math.log(2.0), "log": math.log})


# ---------------------------------------------------------------- golden ----
def test_golden_hand_example_routed(orc):
    g = json.load(open(GOLDEN))["routed"]
    qk = np.array(g["qk"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    mu = np.array(g["mu"], dtype=np.float64)[None]
    inv, idx, margin, _ = orc.route(qk, mu, g["w"])
    assert idx[0, 0].tolist() == g["idx"]
    np.testing.assert_allclose(margin[0, 0], g["margin"], atol=TOL)
    np.testing.assert_allclose(inv[0, 0], [0.2, 0.5, 1.0, 0.2], atol=TOL)
    out, lse, _ = orc.routed_attn(qk, qk, v, idx, _ev(g["scale"]), True)
    want = np.array([[_ev(x) for x in row] for row in g["out"]])
    np.testing.assert_allclose(out[0, 0], want, atol=TOL)
    want_lse = np.array([[_ev(x) for x in row] for row in g["lse"]])
    np.testing.assert_allclose(lse[0, 0], want_lse, atol=TOL)
    mu2 = orc.centroid_update(mu, qk, qk, idx, g["lam"])
    np.testing.assert_allclose(mu2[0], g["mu_new"], atol=TOL)


def test_golden_hand_example_local(orc):
    g = json.load(open(GOLDEN))["local"]
    a = lambda x: np.array(x, dtype=np.float64)[None, None]
    out = orc.local_attn(a(g["q"]), a(g["k"]), a(g["v"]), g["window"], _ev(g["scale"]), True)
    want = np.array([[_ev(x) for x in row] for row in g["out"]])
    np.testing.assert_allclose(out[0, 0], want, atol=TOL)


# ------------------------------------------------------------- O1 and O2 ----
def test_normalize_matches_numpy_norm_and_clamp(orc):
    x = _rng(1).standard_normal((5, 33, 16))
    x[0, 3] = 0.0                                   # zero row: clamp 1e-12
    xhat, inv = orc.normalize(x)
    nrm = np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(inv[nrm > 0], 1.0 / nrm[nrm > 0], rtol=1e-14)
    assert inv[0, 3] == 1e12 and np.all(xhat[0, 3] == 0.0)
    np.testing.assert_allclose(np.linalg.norm(xhat[nrm > 0], axis=-1), 1.0, atol=1e-14)


def test_scores_match_matmul(orc):
    r = _rng(2)
    xhat = _unit(r.standard_normal((50, 8)))
    mu = r.standard_normal((6, 8))
    np.testing.assert_allclose(orc.scores(xhat, mu), mu @ xhat.T, atol=1e-14)


def test_p6_dot_ranking_equals_euclidean_ranking(orc):
    """Summary §2/§4: for unit vectors nearest centroid == largest inner
    product (||x-mu||^2 = 1 - 2<x,mu> + ||mu||^2 with ||mu|| fixed per centroid)."""
    r = _rng(3)
    qk = r.standard_normal((1, 1, 200, 8))
    mu = r.standard_normal((1, 5, 8))
    _, idx, _, _ = orc.route(qk, mu, 20)
    dist = cdist(mu[0], _unit(qk[0, 0]))            # [k, n] Euclidean
    for c in range(5):
        nearest = np.lexsort((np.arange(200), dist[c]))[:20]
        assert sorted(nearest.tolist()) == idx[0, 0, c].tolist()


# -------------------------------------------------------------------- O3 ----
def test_p2_select_structure_and_library_topk(orc):
    r = _rng(4)
    for n, k, w in [(64, 4, 16), (100, 7, 9), (33, 3, 33), (50, 1, 1)]:
        s = r.standard_normal((k, n))
        s[:, ::5] = np.round(s[:, ::5], 1)          # plenty of exact ties
        idx, margin = orc.select(s, w)
        for c in range(k):
            row = idx[c]
            assert np.all(np.diff(row) > 0) and row.min() >= 0 and row.max() < n
            order = np.lexsort((np.arange(n), -s[c]))   # score desc, position asc
            assert row.tolist() == sorted(order[:w].tolist())
            want = np.inf if w == n else s[c, order[w - 1]] - s[c, order[w]]
            assert margin[c] == want
        assert idx.size == k * w


def test_p5_select_brute_force_rank_count(orc):
    """t is chosen iff fewer than w tokens rank strictly above it, where u ranks
    above t when (s_u, -u) > (s_t, -t) lexicographically."""
    r = _rng(5)
    for trial in range(20):
        n, k = int(r.integers(2, 17)), int(r.integers(1, 5))
        w = int(r.integers(1, n + 1))
        s = np.round(r.standard_normal((k, n)), 1)
        idx, _ = orc.select(s, w)
        for c in range(k):
            chosen = []
            for t in range(n):
                above = sum(1 for u in range(n)
                            if s[c, u] > s[c, t] or (s[c, u] == s[c, t] and u < t))
                if above < w:
                    chosen.append(t)
            assert chosen == idx[c].tolist()


def test_p7_membership_invariant_to_centroid_scale(orc):
    r = _rng(6)
    qk = r.standard_normal((2, 2, 128, 16))
    mu = r.standard_normal((2, 8, 16))
    _, idx, _, _ = orc.route(qk, mu, 16)
    for alpha in (0.25, 3.0, 1e3):
        _, idx2, _, _ = orc.route(qk, alpha * mu, 16)
        assert np.array_equal(idx, idx2)


# ----------------------------------------------------------- O4 and O5 ----
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d,scale", [(37, 8, None), (256, 16, 4.0), (1024, 16, None)])
def test_p1_one_cluster_equals_dense_attention(orc, causal, n, d, scale):
    """k=1, w=n: one cluster holding every token is plain (causal) softmax
    attention on the unit-normalised vectors (summary §3)."""
    r = _rng(7)
    q = r.standard_normal((2, 2, n, d))
    kk = r.standard_normal((2, 2, n, d))
    v = r.standard_normal((2, 2, n, d))
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    idx = np.broadcast_to(np.arange(n, dtype=np.int32), (2, 2, 1, n))
    out, lse, _ = orc.routed_attn(q, kk, v, idx, sc, causal)
    qn = F.normalize(torch.from_numpy(q), dim=-1).numpy()
    kn = F.normalize(torch.from_numpy(kk), dim=-1).numpy()
    np.testing.assert_allclose(out, _sdpa(qn, kn, v, sc, causal), atol=1e-12)
    # lse is the log of the softmax denominator
    logits = sc * np.einsum("bhid,bhjd->bhij", qn, kn)
    if causal:
        logits = np.where(np.tril(np.ones((n, n), bool)), logits, -np.inf)
    m = logits.max(-1)
    np.testing.assert_allclose(lse[:, :, 0], m + np.log(np.exp(logits - m[..., None]).sum(-1)),
                               atol=1e-12)


def test_p3_softmax_rows_sum_to_one(orc):
    """With every value row equal to 1, each cluster row returns sum_s P_rs."""
    r = _rng(8)
    qk = r.standard_normal((1, 3, 96, 16))
    mu = r.standard_normal((3, 6, 16))
    _, idx, _, _ = orc.route(qk, mu, 16)
    for scale in (0.25, 4.0, 30.0):
        _, _, oc = orc.routed_attn(qk, qk, np.ones_like(qk), idx, scale, True, want_clusters=True)
        np.testing.assert_allclose(oc, 1.0, atol=TOL)


@pytest.mark.parametrize("causal", [True, False])
def test_p5_attention_brute_force_dense_masks(orc, causal):
    """n <= 16: per cluster, a dense n x n masked softmax over the whole
    sequence (keys outside the cluster, or later than the query when causal,
    get -inf) evaluated by torch SDPA, rows outside the cluster dropped, summed
    over clusters."""
    r = _rng(9)
    for trial in range(10):
        n, k, d = int(r.integers(4, 17)), int(r.integers(1, 5)), 4
        w = int(r.integers(1, n + 1))
        qk = r.standard_normal((1, 1, n, d))
        v = r.standard_normal((1, 1, n, d))
        mu = r.standard_normal((1, k, d))
        _, idx, _, _ = orc.route(qk, mu, w)
        out, _, _ = orc.routed_attn(qk, qk, v, idx, 2.5, causal)
        qn = _unit(qk)
        want = np.zeros((n, d))
        for c in range(k):
            member = np.zeros(n, bool)
            member[idx[0, 0, c]] = True
            allow = member[:, None] & member[None, :]
            if causal:
                allow &= np.tril(np.ones((n, n), bool))
            res = _sdpa(qn, qn, v, 2.5, mask=torch.from_numpy(allow))[0, 0]
            want[member] += res[member]
        np.testing.assert_allclose(out[0, 0], want, atol=1e-12)


def test_p9_outputs_are_convex_combinations(orc):
    r = _rng(10)
    qk = r.standard_normal((1, 2, 200, 16))
    v = r.standard_normal((1, 2, 200, 16))
    mu = r.standard_normal((2, 8, 16))
    _, idx, _, _ = orc.route(qk, mu, 25)
    _, _, oc = orc.routed_attn(qk, qk, v, idx, 3.0, True, want_clusters=True)
    for h in range(2):
        for c in range(8):
            p = idx[0, h, c]
            for rr in range(25):
                seen = v[0, h, p[: rr + 1]]
                assert np.all(oc[0, h, c, rr] <= seen.max(0) + 1e-12)
                assert np.all(oc[0, h, c, rr] >= seen.min(0) - 1e-12)


def test_p12_scatter_zero_and_double_membership(orc):
    r = _rng(11)
    n, d, k, w = 120, 8, 6, 12
    qk = r.standard_normal((1, 1, n, d))
    v = r.standard_normal((1, 1, n, d))
    mu = r.standard_normal((1, k, d))
    _, idx, _, _ = orc.route(qk, mu, w)
    out, _, _ = orc.routed_attn(qk, qk, v, idx, 2.0, True)
    cnt = np.bincount(idx.ravel(), minlength=n)
    assert cnt.sum() == k * w and np.any(cnt == 0) and np.any(cnt == 2)
    assert np.all(out[0, 0, cnt == 0] == 0.0)
    singles = [orc.routed_attn(qk, qk, v, idx[:, :, c:c + 1], 2.0, True)[0] for c in range(k)]
    for t in np.nonzero(cnt == 2)[0]:
        cs = [c for c in range(k) if t in idx[0, 0, c]]
        np.testing.assert_allclose(out[0, 0, t], singles[cs[0]][0, 0, t] + singles[cs[1]][0, 0, t],
                                   atol=1e-12)


def test_distinct_q_and_k_and_unnormalised_mode(orc):
    """normalize=False attends with the vectors as given (used for the pins of
    the backward); with q != k it is SDPA with the two tensors."""
    r = _rng(12)
    q = r.standard_normal((1, 1, 40, 8))
    kk = r.standard_normal((1, 1, 40, 8))
    v = r.standard_normal((1, 1, 40, 8))
    idx = np.arange(40, dtype=np.int32).reshape(1, 1, 1, 40)
    out, _, _ = orc.routed_attn(q, kk, v, idx, 0.7, True, normalize=False)
    np.testing.assert_allclose(out, _sdpa(q, kk, v, 0.7, True), atol=1e-12)


# -------------------------------------------------------------------- O6 ----
def test_p4_ema_closed_forms(orc):
    r = _rng(13)
    B, H, n, d, k, w = 3, 2, 64, 8, 4, 16
    qk = r.standard_normal((B, H, n, d))
    mu = r.standard_normal((H, k, d))
    _, idx, _, _ = orc.route(qk, mu, w)
    assert np.array_equal(orc.centroid_update(mu, qk, qk, idx, 1.0), mu)
    # lam = 0: (S_Q + S_K)/2 with S the batch-wide member sums of x^
    xh = _unit(qk)
    S = np.zeros((H, k, d))
    for b in range(B):
        for h in range(H):
            for c in range(k):
                S[h, c] += xh[b, h, idx[b, h, c]].sum(0)
    np.testing.assert_allclose(orc.centroid_update(mu, qk, qk, idx, 0.0), S, atol=1e-12)
    # all members equal u (shared q = k): lam*mu + (1-lam)*B*w*u
    u = _unit(r.standard_normal(d))
    same = np.broadcast_to(3.7 * u, (B, H, n, d)).copy()
    got = orc.centroid_update(mu, same, same, idx, 0.9)
    np.testing.assert_allclose(got, 0.9 * mu + 0.1 * B * w * u, atol=1e-12)
    # T updates with a fixed membership: lam^T mu0 + (1 - lam^T) S
    m = mu.copy()
    for _ in range(7):
        m = orc.centroid_update(m, qk, qk, idx, 0.8)
    np.testing.assert_allclose(m, 0.8 ** 7 * mu + (1 - 0.8 ** 7) * S, atol=1e-12)
    # distinct q and k: lam*mu + (1-lam)/2 (S_Q + S_K)
    kk = r.standard_normal((B, H, n, d))
    SK = np.zeros((H, k, d))
    xk = _unit(kk)
    for b in range(B):
        for h in range(H):
            for c in range(k):
                SK[h, c] += xk[b, h, idx[b, h, c]].sum(0)
    np.testing.assert_allclose(orc.centroid_update(mu, qk, kk, idx, 0.3),
                               0.3 * mu + 0.35 * (S + SK), atol=1e-12)


def test_p11_ema_sum_order_vs_exact_sum(orc):
    r = _rng(14)
    B, H, n, d, k, w = 8, 1, 256, 16, 4, 64
    qk = r.standard_normal((B, H, n, d))
    mu = r.standard_normal((H, k, d))
    _, idx, _, _ = orc.route(qk, mu, w)
    got = orc.centroid_update(mu, qk, qk, idx, 0.0)
    xh = _unit(qk)
    for c in range(k):
        for i in range(d):
            terms = [xh[b, 0, t, i] for b in range(B) for t in idx[b, 0, c]]
            assert abs(got[0, c, i] - math.fsum(terms)) < 1e-12


# -------------------------------------------------------------------- O7 ----
@pytest.mark.parametrize("n,window", [(50, 1), (50, 7), (50, 50), (50, 80), (300, 64)])
def test_p8_local_against_banded_sdpa(orc, n, window):
    r = _rng(15)
    q, kk, v = (r.standard_normal((2, 3, n, 8)) for _ in range(3))
    out = orc.local_attn(q, kk, v, window, 0.9, True)
    i = np.arange(n)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - window)
    np.testing.assert_allclose(out, _sdpa(q, kk, v, 0.9, mask=torch.from_numpy(band)), atol=1e-12)
    if window == 1:
        np.testing.assert_allclose(out, v, atol=1e-14)
    if window >= n:
        np.testing.assert_allclose(out, _sdpa(q, kk, v, 0.9, True), atol=1e-12)


def test_local_non_causal_band(orc):
    r = _rng(16)
    n, window = 40, 5
    q, kk, v = (r.standard_normal((1, 1, n, 4)) for _ in range(3))
    out = orc.local_attn(q, kk, v, window, 1.1, False)
    i = np.arange(n)
    band = np.abs(i[None, :] - i[:, None]) < window
    np.testing.assert_allclose(out, _sdpa(q, kk, v, 1.1, mask=torch.from_numpy(band)), atol=1e-12)


# -------------------------------------------------------------------- O8 ----
def test_p10_backward_matches_autograd_dense(orc):
    """k=1, w=n: gradients of causal SDPA on the normalised vectors, by torch
    autograd in float64 (normalisation held fixed, as in O8)."""
    r = _rng(17)
    n, d = 48, 8
    q, kk, v, g = (r.standard_normal((1, 2, n, d)) for _ in range(4))
    idx = np.broadcast_to(np.arange(n, dtype=np.int32), (1, 2, 1, n))
    dq, dk, dv = orc.routed_attn_bwd(q, kk, v, idx, g, 1.3, True)
    tq = torch.from_numpy(_unit(q)).requires_grad_()
    tk = torch.from_numpy(_unit(kk)).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=1.3)
    o.backward(torch.from_numpy(g))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_p10_backward_finite_differences_routed(orc):
    """Several overlapping clusters (fixed membership): central differences of
    L = <dout, out> with respect to q^, k^ and v, evaluated with the oracle's
    forward on unnormalised inputs (normalize=False, so the inputs are q^)."""
    r = _rng(18)
    n, d, k, w = 20, 4, 3, 8
    q = _unit(r.standard_normal((1, 1, n, d)))
    kk = _unit(r.standard_normal((1, 1, n, d)))
    v = r.standard_normal((1, 1, n, d))
    g = r.standard_normal((1, 1, n, d))
    mu = r.standard_normal((1, k, d))
    _, idx, _, _ = orc.route(q, mu, w)
    dq, dk, dv = orc.routed_attn_bwd(q, kk, v, idx, g, 1.7, True)

    def loss(qq, kq, vv):
        o, _, _ = orc.routed_attn(qq, kq, vv, idx, 1.7, True, normalize=False)
        return float((o * g).sum())

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        args = [q, kk, v]
        num = np.zeros_like(q)
        for t in range(n):
            for i in range(d):
                a = [x.copy() for x in args]
                b = [x.copy() for x in args]
                a[which][0, 0, t, i] += h
                b[which][0, 0, t, i] -= h
                num[0, 0, t, i] = (loss(*a) - loss(*b)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


# ---- the layer stack (projections, rounding, one layer) --------------------------------

def test_round_bf16_ties_and_values(orc):
    """bfloat16 keeps 8 significant bits; halfway cases go to the even one."""
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7, 1 + 2 ** -9, -(1 + 2 ** -8),
                  3 * 2 ** -130, 255.0, 257.0, 0.0])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, 1.0, -1.0, 3 * 2 ** -130, 255.0, 256.0,
                     0.0])
    np.testing.assert_array_equal(orc.round_bf16(x), want)


def test_round_bf16_matches_torch_on_float32_values(orc):
    """On float32-representable inputs it equals torch's float32 -> bfloat16
    conversion (round to nearest even), an independent implementation."""
    rng = np.random.default_rng(3)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(f).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(orc.round_bf16(f.astype(np.float64)), want)


def test_in_proj_identity_splits_heads(orc):
    """With W_in = I the projections are x's columns, split into head-major
    tensors in the order qk, v, q_l, k_l, v_l (exact: x is bf16 already)."""
    B, n, d, R, L = 2, 5, 4, 2, 1
    dm = (2 * R + 3 * L) * d
    x = orc.round_bf16(np.random.default_rng(4).standard_normal((B, n, dm)))
    outs = orc.in_proj(x, np.eye(dm), R, L, d)
    heads = [(0, R), (R, 2 * R), (2 * R, 2 * R + L), (2 * R + L, 2 * R + 2 * L),
             (2 * R + 2 * L, 2 * R + 3 * L)]
    for t, (h0, h1) in zip(outs, heads):
        for b in range(B):
            for h in range(h0, h1):
                np.testing.assert_array_equal(t[b, h - h0], x[b, :, h * d:(h + 1) * d])
    assert orc.in_proj(x[:, :, :2 * R * d], np.eye(2 * R * d), R, 0, d)[2] is None


def test_in_proj_is_rounded_exact_product(orc):
    rng = np.random.default_rng(5)
    x = orc.round_bf16(rng.standard_normal((1, 7, 16)))
    w = orc.round_bf16(rng.standard_normal((2 * 16, 16)))
    qk, v, _, _, _ = orc.in_proj(x, w, 1, 0, 16)
    exact = np.einsum("tk,nk->tn", x[0], w)   # independent of the oracle's product
    np.testing.assert_array_equal(qk[0, 0], orc.round_bf16(exact[:, :16]))
    np.testing.assert_array_equal(v[0, 0], orc.round_bf16(exact[:, 16:]))


def test_out_proj_zero_weights_and_concat_order(orc):
    rng = np.random.default_rng(6)
    B, n, d, R, L = 2, 3, 4, 2, 1
    o_r = orc.round_bf16(rng.standard_normal((B, R, n, d)))
    o_l = orc.round_bf16(rng.standard_normal((B, L, n, d)))
    dm = (R + L) * d
    x = orc.round_bf16(rng.standard_normal((B, n, dm)))
    np.testing.assert_array_equal(orc.out_proj(o_r, o_l, np.zeros((dm, dm)), x), x)
    y = orc.out_proj(o_r, o_l, np.eye(dm))                  # identity: the concatenation
    for b in range(B):
        for h in range(R + L):
            src = o_r[b, h] if h < R else o_l[b, h - R]
            np.testing.assert_array_equal(y[b, :, h * d:(h + 1) * d], src)


def test_layer_forward_composition_and_zero_output_map(orc):
    """One layer with W_o = 0 leaves x unchanged, and its centroid update is
    that of its own routed projections."""
    rng = np.random.default_rng(8)
    B, n, dm, d, R, L, k, w = 1, 40, 16, 16, 1, 1, 3, 10
    x = orc.round_bf16(rng.standard_normal((B, n, dm)))
    w_in = orc.round_bf16(rng.standard_normal(((2 * R + 3 * L) * d, dm)) / 4)
    mu = rng.standard_normal((R, k, d))
    res = orc.layer_forward(x, w_in, np.zeros((dm, (R + L) * d)), mu, R, L, d, w, 8, 0.9)
    np.testing.assert_array_equal(res["y"], x)
    qk = orc.in_proj(x, w_in, R, L, d)[0]
    np.testing.assert_allclose(res["mu"], orc.centroid_update(mu, qk, qk, res["idx"], 0.9),
                               rtol=0, atol=1e-12)
    assert res["o_r"].shape == (B, R, n, d) and res["o_l"].shape == (B, L, n, d)


# ---- the layer's backward (O9, the normalisation, the projections) ----------------------

def _band(n, window, causal):
    i = np.arange(n)
    if causal:
        return (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - window)
    return np.abs(i[None, :] - i[:, None]) < window


@pytest.mark.parametrize("n,window,causal", [(30, 7, True), (12, 12, True), (25, 1, True),
                                             (20, 4, False)])
def test_p13_local_bwd_matches_autograd_banded(orc, n, window, causal):
    """O9 against torch autograd (float64) of SDPA with the same band."""
    r = _rng(30)
    q, kk, v, g = (r.standard_normal((2, 2, n, 6)) for _ in range(4))
    dq, dk, dv = orc.local_attn_bwd(q, kk, v, g, window, 0.8, causal)
    t = [torch.from_numpy(a.copy()).requires_grad_() for a in (q, kk, v)]
    o = F.scaled_dot_product_attention(*t, attn_mask=torch.from_numpy(_band(n, window, causal)),
                                       scale=0.8)
    o.backward(torch.from_numpy(g))
    for got, ref in zip((dq, dk, dv), t):
        np.testing.assert_allclose(got, ref.grad.numpy(), atol=1e-11)


def test_local_bwd_finite_differences(orc):
    """Central differences of <g, local_attn(q, k, v)>, brute force."""
    r = _rng(31)
    n, d, window = 9, 3, 4
    q, kk, v, g = (r.standard_normal((1, 1, n, d)) for _ in range(4))
    grads = orc.local_attn_bwd(q, kk, v, g, window, 1.2, True)
    h = 1e-6
    for which in range(3):
        num = np.zeros_like(q)
        for t in range(n):
            for i in range(d):
                a = [q.copy(), kk.copy(), v.copy()]
                b = [q.copy(), kk.copy(), v.copy()]
                a[which][0, 0, t, i] += h
                b[which][0, 0, t, i] -= h
                num[0, 0, t, i] = ((orc.local_attn(*a, window, 1.2, True) * g).sum()
                                   - (orc.local_attn(*b, window, 1.2, True) * g).sum()) / (2 * h)
        np.testing.assert_allclose(grads[which], num, rtol=1e-6, atol=1e-8)


def test_normalize_bwd_matches_autograd_and_clamp(orc):
    r = _rng(32)
    x = r.standard_normal((3, 5, 7))
    x[1, 2] = 0.0                                      # clamped row: r = 1e-12 is constant
    g = r.standard_normal(x.shape)
    tx = torch.from_numpy(x.copy()).requires_grad_()
    nrm = torch.clamp(torch.linalg.vector_norm(tx, dim=-1, keepdim=True), min=1e-12)
    (tx / nrm).backward(torch.from_numpy(g))
    got = orc.normalize_bwd(x, g)
    np.testing.assert_allclose(got, tx.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(got[1, 2], g[1, 2] / 1e-12)
    # the gradient is orthogonal to x (scaling x does not change x^)
    keep = np.ones(x.shape[:-1], bool)
    keep[1, 2] = False
    assert np.abs((got * x).sum(-1)[keep]).max() < 1e-12


def test_proj_bwd_matches_autograd(orc):
    """Both projections' gradients (rounding=False) against torch autograd of
    the exact linear maps, including the residual's gradient."""
    r = _rng(33)
    B, n, d, R, L = 2, 3, 4, 2, 1
    dm = 10
    x = r.standard_normal((B, n, dm))
    w_in = r.standard_normal(((2 * R + 3 * L) * d, dm))
    w_o = r.standard_normal((dm, (R + L) * d))
    o_r, o_l = r.standard_normal((B, R, n, d)), r.standard_normal((B, L, n, d))
    dy = r.standard_normal((B, n, dm))
    tr, tl, tw = (torch.from_numpy(a.copy()).requires_grad_() for a in (o_r, o_l, w_o))
    cat = torch.cat([tr, tl], 1).permute(0, 2, 1, 3).reshape(B, n, -1)
    (cat @ tw.T).backward(torch.from_numpy(dy))
    do_r, do_l, dw_o = orc.out_proj_bwd(dy, o_r, o_l, w_o, rounding=False)
    np.testing.assert_allclose(do_r, tr.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(do_l, tl.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dw_o, tw.grad.numpy(), atol=1e-12)
    gh = [r.standard_normal((B, h, n, d)) for h in (R, R, L, L, L)]
    tx, twi = (torch.from_numpy(a.copy()).requires_grad_() for a in (x, w_in))
    y = (tx @ twi.T).reshape(B, n, 2 * R + 3 * L, d).permute(0, 2, 1, 3)
    g = torch.from_numpy(np.concatenate(gh, axis=1))
    ((y * g).sum() + (tx * torch.from_numpy(dy)).sum()).backward()
    dx, dw_in = orc.in_proj_bwd(x, w_in, *gh, dy=dy, rounding=False)
    np.testing.assert_allclose(dx, tx.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dw_in, twi.grad.numpy(), atol=1e-12)
    # rounding=True rounds the heads' gradients (the products' operands) only
    dx_r, _ = orc.in_proj_bwd(x, w_in, *[orc.round_bf16(a) for a in gh], rounding=True)
    dx_e, _ = orc.in_proj_bwd(x, w_in, *[orc.round_bf16(a) for a in gh], rounding=False)
    np.testing.assert_array_equal(dx_r, dx_e)


def test_layer_backward_matches_autograd(orc):
    """The whole layer (fixed membership, no storage rounding) in torch float64:
    projections, normalised shared q/k, per-cluster causal attention scattered
    back, banded local attention; autograd of <dy, y> against layer_backward."""
    r = _rng(34)
    B, n, dm, d, R, L, k, w, window = 1, 24, 12, 4, 1, 1, 3, 9, 5
    sc = 0.7
    x = r.standard_normal((B, n, dm))
    w_in = r.standard_normal(((2 * R + 3 * L) * d, dm)) / 3
    w_o = r.standard_normal((dm, (R + L) * d)) / 3
    mu = r.standard_normal((R, k, d))
    dy = r.standard_normal((B, n, dm))
    heads = (x.reshape(B * n, dm) @ w_in.T).reshape(B, n, 2 * R + 3 * L, d).transpose(0, 2, 1, 3)
    qk, v = heads[:, :R].copy(), heads[:, R:2 * R].copy()
    ql, kl, vl = heads[:, 2 * R:2 * R + L].copy(), heads[:, 2 * R + L:2 * R + 2 * L].copy(), \
        heads[:, 2 * R + 2 * L:].copy()
    _, idx, _, _ = orc.route(qk, mu, w)
    o_r, _, _ = orc.routed_attn(qk, qk, v, idx, sc, True, True)
    o_l = orc.local_attn(ql, kl, vl, window, sc, True)
    fwd = {"qk": qk, "v": v, "q_l": ql, "k_l": kl, "v_l": vl, "idx": idx, "o_r": o_r, "o_l": o_l}
    got = orc.layer_backward(x, w_in, w_o, fwd, dy, R, L, d, window, sc, rounding=False)

    tx, twi, two = (torch.from_numpy(a.copy()).requires_grad_() for a in (x, w_in, w_o))
    hh = (tx.reshape(B * n, dm) @ twi.T).reshape(B, n, 2 * R + 3 * L, d).permute(0, 2, 1, 3)
    tqk, tv = hh[:, :R], hh[:, R:2 * R]
    tq, tkl, tvl = hh[:, 2 * R:2 * R + L], hh[:, 2 * R + L:2 * R + 2 * L], hh[:, 2 * R + 2 * L:]
    qn = tqk / torch.clamp(torch.linalg.vector_norm(tqk, dim=-1, keepdim=True), min=1e-12)
    outs = []
    for b in range(B):
        for h in range(R):
            acc = torch.zeros((n, d), dtype=torch.float64)
            for c in range(k):
                p = torch.from_numpy(idx[b, h, c].astype(np.int64))
                qc, vc = qn[b, h][p], tv[b, h][p]
                vis = p[None, :] <= p[:, None]
                o = F.scaled_dot_product_attention(qc[None], qc[None], vc[None],
                                                   attn_mask=vis[None], scale=sc)[0]
                acc = acc.index_add(0, p, o)
            outs.append(acc)
    t_or = torch.stack(outs).reshape(B, R, n, d)
    t_ol = F.scaled_dot_product_attention(tq, tkl, tvl,
                                          attn_mask=torch.from_numpy(_band(n, window, True)),
                                          scale=sc)
    cat = torch.cat([t_or, t_ol], 1).permute(0, 2, 1, 3).reshape(B, n, -1)
    y = tx + cat @ two.T
    (y * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(got["dx"], tx.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(got["dw_in"], twi.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(got["dw_o"], two.grad.numpy(), atol=1e-10)


# ---- variants: blocked local attention, nearest-centroid assignment, partition ---------

def _block_mask(n, block, lookback):
    i = np.arange(n)
    lo = np.maximum(0, (i // block - lookback) * block)
    return (i[None, :] <= i[:, None]) & (i[None, :] >= lo[:, None])


@pytest.mark.parametrize("n,block,lookback", [(40, 8, 1), (37, 5, 0), (30, 7, 2), (20, 32, 0)])
def test_o10_blocked_against_masked_sdpa(orc, n, block, lookback):
    r = _rng(40)
    q, kk, v = (r.standard_normal((2, 2, n, 6)) for _ in range(3))
    out = orc.local_attn_blocked(q, kk, v, block, lookback, 0.8)
    mask = torch.from_numpy(_block_mask(n, block, lookback))
    np.testing.assert_allclose(out, _sdpa(q, kk, v, 0.8, mask=mask), atol=1e-12)
    if block >= n and lookback == 0:                 # one block: plain causal attention
        np.testing.assert_allclose(out, _sdpa(q, kk, v, 0.8, True), atol=1e-12)


def test_o10_block_of_one_is_identity(orc):
    r = _rng(41)
    q, kk, v = (r.standard_normal((1, 1, 15, 4)) for _ in range(3))
    np.testing.assert_allclose(orc.local_attn_blocked(q, kk, v, 1, 0, 1.0), v, atol=1e-14)


def test_o11_argmax_is_nearest_centroid(orc):
    """For unit tokens and unit centroids the largest inner product is the
    smallest Euclidean distance (scipy cdist, an independent route)."""
    r = _rng(42)
    x = r.standard_normal((2, 3, 50, 8))
    mu = _unit(r.standard_normal((3, 7, 8)))
    label, margin = orc.argmax_labels(x, mu)
    xh = _unit(x)
    for b in range(2):
        for h in range(3):
            dist = cdist(xh[b, h], mu[h])
            np.testing.assert_array_equal(label[b, h], np.argmin(dist, axis=1))
            srt = np.sort(xh[b, h] @ mu[h].T, axis=1)
            np.testing.assert_allclose(margin[b, h], srt[:, -1] - srt[:, -2], atol=1e-12)


def test_o11_argmax_ties_to_lower_index(orc):
    x = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    mu = np.array([[[1.0, 0.0], [1.0, 0.0], [0.0, 1.0]]])      # centroids 0 and 1 equal
    label, margin = orc.argmax_labels(x, mu)
    np.testing.assert_array_equal(label[0, 0], [0, 2])
    assert margin[0, 0, 0] == 0.0


def test_o11_ema_with_one_centroid_is_the_full_membership(orc):
    """k = 1: every token is assigned to the only centroid, as O6 with w = n."""
    r = _rng(43)
    q, kk = r.standard_normal((2, 2, 30, 5)), r.standard_normal((2, 2, 30, 5))
    mu = r.standard_normal((2, 1, 5))
    idx = np.broadcast_to(np.arange(30, dtype=np.int32), (2, 2, 1, 30))
    np.testing.assert_allclose(orc.centroid_update_argmax(mu, q, kk, 0.8),
                               orc.centroid_update(mu, q, kk, idx, 0.8), atol=1e-12)


def test_o11_ema_hand_example(orc):
    """Two 2-d tokens, two centroids: token 0 is nearest to centroid 0, token 1
    to centroid 1; with q = k, mu_c <- lam mu_c + (1 - lam) x^_c."""
    x = np.array([[[[3.0, 0.0], [0.0, -2.0]]]])
    mu = np.array([[[1.0, 0.0], [0.0, -1.0]]])
    got = orc.centroid_update_argmax(mu, x, x, 0.75)
    np.testing.assert_allclose(got, [[[1.0, 0.0], [0.0, -1.0]]], atol=1e-15)
    mu2 = np.array([[[0.6, 0.8], [0.0, -1.0]]])
    got2 = orc.centroid_update_argmax(mu2, x, x, 0.5)
    np.testing.assert_allclose(got2, [[[0.8, 0.4], [0.0, -1.0]]], atol=1e-15)


def test_o12_partition_invariants_and_balanced_case(orc):
    r = _rng(44)
    n, k, d = 48, 4, 6
    x = r.standard_normal((2, 2, n, d))
    mu = _unit(r.standard_normal((2, k, d)))
    idx = orc.route_partition(x, mu)
    assert idx.shape == (2, 2, k, n // k)
    for b in range(2):
        for h in range(2):
            np.testing.assert_array_equal(np.sort(idx[b, h].ravel()), np.arange(n))
            assert np.all(np.diff(idx[b, h], axis=1) > 0)
    # tokens built so that each centroid is the nearest one of exactly n/k tokens
    cent = _unit(r.standard_normal((k, d)))
    toks = np.repeat(cent, n // k, axis=0) + 0.01 * r.standard_normal((n, d))
    perm = r.permutation(n)
    xb = toks[perm][None, None]
    got = orc.route_partition(xb, cent[None])
    lab = np.argmin(cdist(_unit(xb[0, 0]), cent), axis=1)
    for c in range(k):
        np.testing.assert_array_equal(got[0, 0, c], np.flatnonzero(lab == c))


def test_o12_partition_hand_example(orc):
    """All four tokens prefer centroid 0: its cluster takes the two with the
    largest scores against it, centroid 1 the other two."""
    x = np.array([[[[1.0, 0.1], [1.0, 0.5], [1.0, 0.0], [1.0, 0.3]]]])
    mu = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    idx = orc.route_partition(x, mu)
    np.testing.assert_array_equal(idx[0, 0], [[0, 2], [1, 3]])


# ---- incremental decode --------------------------------------------------------------------

def test_decode_one_cluster_is_dense_causal_attention(orc):
    """k = 1: the only cluster holds every earlier token, so decoding position
    t equals row t of causal SDPA over the normalised vectors."""
    r = _rng(50)
    B, H, n, d = 1, 2, 24, 8
    x = r.standard_normal((B, H, n, d))
    v = r.standard_normal((B, H, n, d))
    mu = r.standard_normal((H, 1, d))
    t = 17
    idx = np.broadcast_to(np.arange(t, dtype=np.int32), (B, H, 1, t))
    cache = orc.decode_cache_from_prefill(x[:, :, :t], v[:, :, :t], idx, 32)
    out, label, cache2 = orc.decode_step(cache, x[:, :, t], v[:, :, t], t, mu, 0.6)
    want = _sdpa(_unit(x[:, :, :t + 1]), _unit(x[:, :, :t + 1]), v[:, :, :t + 1], 0.6, True)[:, :, t]
    np.testing.assert_allclose(out, want, atol=1e-12)
    assert np.all(label == 0) and np.all(cache2["len"] == t + 1)
    assert np.all(cache2["pos"][:, :, 0, t] == t)


def test_decode_routes_to_nearest_centroid_and_attends_its_cache(orc):
    r = _rng(51)
    B, H, n, d, k, w = 2, 1, 40, 6, 4, 10
    x = r.standard_normal((B, H, n, d))
    v = r.standard_normal((B, H, n, d))
    mu = _unit(r.standard_normal((H, k, d)))
    _, idx, _, _ = orc.route(x[:, :, :n - 1], mu, w)
    cache = orc.decode_cache_from_prefill(x[:, :, :n - 1], v[:, :, :n - 1], idx, w + 4)
    out, label, cache2 = orc.decode_step(cache, x[:, :, n - 1], v[:, :, n - 1], n - 1, mu, 1.1)
    for b in range(B):
        c = int(np.argmin(cdist(_unit(x[b, 0, n - 1][None]), mu[0])))
        assert label[b, 0] == c
        members = list(idx[b, 0, c]) + [n - 1]
        q = _unit(x[b, 0, members])
        want = _sdpa(q[None, None], q[None, None], v[b, 0, members][None, None], 1.1, True)[0, 0, -1]
        np.testing.assert_allclose(out[b, 0], want, atol=1e-12)


def test_local_decode_matches_local_attention(orc):
    """Feeding a sequence one token at a time through the ring buffer gives
    the rows of O7 (the C sliding-window attention)."""
    r = _rng(52)
    B, H, n, d, W = 1, 2, 30, 5, 7
    q, kk, v = (r.standard_normal((B, H, n, d)) for _ in range(3))
    want = orc.local_attn(q, kk, v, W, 0.9, True)
    rk, rv = np.zeros((B, H, W, d)), np.zeros((B, H, W, d))
    for t in range(n):
        out, rk, rv = orc.local_decode_step(rk, rv, q[:, :, t], kk[:, :, t], v[:, :, t], t, W, 0.9)
        np.testing.assert_allclose(out, want[:, :, t], atol=1e-12)


def test_decode_ties_to_lower_centroid(orc):
    """Two equal centroids: the new token joins the lower-indexed one (and its
    cache), as the nearest-centroid rule breaks ties."""
    B, H, d = 1, 1, 3
    mu = np.array([[[0.0, 0.0, 1.0], [1.0, 0.0, 0.0], [1.0, 0.0, 0.0]]])
    x = np.array([[[[0.0, 0.0, 2.0], [3.0, 0.5, 0.0], [0.1, 0.0, 4.0], [2.0, -0.5, 0.0]]]])
    v = np.arange(12, dtype=float).reshape(B, H, 4, d)
    idx = np.array([[[[0], [1], [1]]]], dtype=np.int32)      # clusters 1 and 2 both hold token 1
    cache = orc.decode_cache_from_prefill(x[:, :, :3], v[:, :, :3], idx, 4)
    out, label, cache2 = orc.decode_step(cache, x[:, :, 3], v[:, :, 3], 3, mu, 1.0)
    assert label[0, 0] == 1
    np.testing.assert_array_equal(cache2["len"][0, 0], [1, 2, 1])
    q = _unit(x[0, 0, [1, 3]])
    want = _sdpa(q[None, None], q[None, None], v[0, 0, [1, 3]][None, None], 1.0, True)[0, 0, -1]
    np.testing.assert_allclose(out[0, 0], want, atol=1e-12)


def test_decode_given_label_joins_that_cluster(orc):
    """With the two equal centroids above, the step told to take the upper one
    appends to that cluster's cache and attends to its members instead; told
    its own choice, it changes nothing."""
    B, H, d = 1, 1, 3
    mu = np.array([[[0.0, 0.0, 1.0], [1.0, 0.0, 0.0], [1.0, 0.0, 0.0]]])
    x = np.array([[[[0.0, 0.0, 2.0], [3.0, 0.5, 0.0], [0.1, 0.0, 4.0], [2.0, -0.5, 0.0]]]])
    v = np.arange(12, dtype=float).reshape(B, H, 4, d)
    idx = np.array([[[[0], [1], [2]]]], dtype=np.int32)
    cache = orc.decode_cache_from_prefill(x[:, :, :3], v[:, :, :3], idx, 4)
    out1, lab1, c1 = orc.decode_step(cache, x[:, :, 3], v[:, :, 3], 3, mu, 1.0)
    out2, lab2, c2 = orc.decode_step(cache, x[:, :, 3], v[:, :, 3], 3, mu, 1.0,
                                     label_given=np.array([[1]]))
    assert lab1[0, 0] == 1 and lab2[0, 0] == 1
    np.testing.assert_array_equal(out1, out2)
    for name in c1:
        np.testing.assert_array_equal(c1[name], c2[name])
    out3, lab3, c3 = orc.decode_step(cache, x[:, :, 3], v[:, :, 3], 3, mu, 1.0,
                                     label_given=np.array([[2]]))
    assert lab3[0, 0] == 2
    np.testing.assert_array_equal(c3["len"][0, 0], [1, 1, 2])
    assert c3["pos"][0, 0, 2, 1] == 3
    q = _unit(x[0, 0, [2, 3]])
    want = _sdpa(q[None, None], q[None, None], v[0, 0, [2, 3]][None, None], 1.0, True)[0, 0, -1]
    np.testing.assert_allclose(out3[0, 0], want, atol=1e-12)


# ---- separately routed queries and keys ---------------------------------------------------

def test_split_with_one_membership_is_noncausal_routed_attention(orc):
    """The same membership on both sides: the C routed attention (non-causal)."""
    r = _rng(60)
    B, H, n, d, k, w = 2, 2, 40, 8, 4, 12
    q, kk, v = (r.standard_normal((B, H, n, d)) for _ in range(3))
    mu = _unit(r.standard_normal((H, k, d)))
    _, idx, _, _ = orc.route(q, mu, w)
    out, lse, _, _ = orc.routed_attn_split(q, kk, v, idx, idx, 0.7)
    want, want_lse, _ = orc.routed_attn(q, kk, v, idx, 0.7, causal=False)
    np.testing.assert_allclose(out, want, atol=1e-12)
    np.testing.assert_allclose(lse, want_lse, atol=1e-12)


def test_split_one_cluster_of_everything_is_dense_attention(orc):
    """k = 1, w = n on both sides: non-causal SDPA of the unit queries on the unit keys."""
    r = _rng(61)
    B, H, n, d = 1, 2, 20, 6
    q, kk, v = (r.standard_normal((B, H, n, d)) for _ in range(3))
    idx = np.broadcast_to(np.arange(n, dtype=np.int32), (B, H, 1, n))
    out, _, sum_q, sum_k = orc.routed_attn_split(q, kk, v, idx, idx[:, :, :, ::-1].copy()[:, :, :, ::-1], 1.3)
    want = _sdpa(_unit(q), _unit(kk), v, 1.3, False)
    np.testing.assert_allclose(out, want, atol=1e-12)
    np.testing.assert_allclose(sum_q[:, :, 0], _unit(q).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(sum_k[:, :, 0], _unit(kk).sum(axis=2), atol=1e-12)


def test_split_hand_example(orc):
    """Token 0's only cluster has the single key token 2: out[0] = v[2]; token 1
    is in two query clusters: the sum of both rows; token 3 is in none: 0."""
    d = 2
    q = np.array([[[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [0.5, -1.0]]]])
    kk = np.array([[[[1.0, 0.0], [0.0, 2.0], [3.0, 0.0], [0.0, -1.0]]]])
    v = np.array([[[[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]]]])
    idx_q = np.array([[[[0, 1], [1, 2]]]], dtype=np.int32)
    idx_k = np.array([[[[2, 2], [1, 3]]]], dtype=np.int32)
    out, lse, _, _ = orc.routed_attn_split(q, kk, v, idx_q, idx_k, 1.0)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 2], atol=1e-12)
    # token 1: cluster 0 (keys 2, 2 -> v[2]) plus cluster 1 (keys 1 and 3, logits +1 and -1)
    p = np.exp([1.0, -1.0]) / np.exp([1.0, -1.0]).sum()
    np.testing.assert_allclose(out[0, 0, 1], v[0, 0, 2] + p[0] * v[0, 0, 1] + p[1] * v[0, 0, 3],
                               atol=1e-12)
    np.testing.assert_array_equal(out[0, 0, 3], np.zeros(d))
    np.testing.assert_allclose(lse[0, 0, 0, 0], 1.0 + np.log(2.0), atol=1e-12)   # logit 1, twice


# ---- Jensen-Shannon divergence between local and routed attention --------------------------

def _dense_js(p, q):
    from scipy.spatial.distance import jensenshannon
    return jensenshannon(p, q) ** 2          # natural log by default; scipy returns the root


def test_js_matches_scipy_on_dense_distributions(orc):
    """Each row's divergence against scipy's Jensen-Shannon distance (squared) of
    the two distributions built here by brute force (masked softmax rows)."""
    r = _rng(70)
    B, H, n, d, k, w, W = 1, 2, 30, 6, 3, 8, 5
    qk = r.standard_normal((B, H, n, d))
    ql, kl = r.standard_normal((B, H, n, d)), r.standard_normal((B, H, n, d))
    mu = _unit(r.standard_normal((H, k, d)))
    _, idx, _, _ = orc.route(qk, mu, w)
    js = orc.attn_js(qk, idx, ql, kl, W, 1.7, 0.4)
    u = _unit(qk)
    for b in range(B):
        for h in range(H):
            for c in range(k):
                for rr in range(w):
                    i = idx[b, h, c, rr]
                    lo = max(0, i - W + 1)
                    p = np.zeros(n)
                    p[lo:i + 1] = _softmax(0.4 * kl[b, h, lo:i + 1] @ ql[b, h, i])
                    keys = idx[b, h, c, :rr + 1]
                    q = np.zeros(n)
                    q[keys] = _softmax(1.7 * u[b, h, keys] @ u[b, h, i])
                    assert abs(js[b, h, c, rr] - _dense_js(p, q)) < 1e-12


def test_js_zero_for_identical_and_bounded(orc):
    """One cluster of every token, a window covering the sequence and the local
    head given the routed head's unit vectors and scale: P = Q, JS = 0.  For
    random inputs 0 <= JS <= ln 2."""
    r = _rng(71)
    B, H, n, d = 1, 1, 16, 4
    qk = r.standard_normal((B, H, n, d))
    idx = np.broadcast_to(np.arange(n, dtype=np.int32), (B, H, 1, n))
    u = _unit(qk)
    js = orc.attn_js(qk, idx, u, u, n, 0.9, 0.9)
    np.testing.assert_allclose(js, 0.0, atol=1e-13)
    ql, kl = 5 * r.standard_normal((B, H, n, d)), 5 * r.standard_normal((B, H, n, d))
    js2 = orc.attn_js(qk, idx, ql, kl, 3, 4.0, 1.0)
    assert np.all(js2 >= -1e-15) and np.all(js2 <= np.log(2) + 1e-15)


def test_js_window_of_one_closed_form(orc):
    """Window 1: P is the query itself.  With Q = (q_j, q_i) over an earlier key
    j and the query: JS = 1/2 ln(2/(1+q_i)) + 1/2 (q_i ln(2 q_i/(1+q_i)) + q_j ln 2)."""
    qk = np.array([[[[1.0, 0.0], [0.6, 0.8]]]])
    idx = np.array([[[[0, 1]]]], dtype=np.int32)
    ql = np.ones((1, 1, 2, 2))
    js = orc.attn_js(qk, idx, ql, ql, 1, 2.0, 1.0)
    s = 2.0 * np.array([0.6, 1.0])           # logits of key 0 and of the query itself
    qj, qi = np.exp(s) / np.exp(s).sum()
    want = 0.5 * np.log(2 / (1 + qi)) + 0.5 * (qi * np.log(2 * qi / (1 + qi)) + qj * np.log(2))
    assert abs(js[0, 0, 0, 1] - want) < 1e-13
    assert abs(js[0, 0, 0, 0]) < 1e-13       # the first token sees only itself on both sides
