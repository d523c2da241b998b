"""Helpers shared by the tests: device transfer of synthetic inputs and the
comparison rules between the HIP path and the oracle."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances (the arithmetic is float32 on the device, float64 in the oracle).
MARGIN = 1e-5            # memberships must match wherever the top-w score gap exceeds this
F32_MAX_ABS = 1e-4       # float32 outputs
BF16_MAX_ABS = 2e-2      # bfloat16 outputs
BF16_MEAN_REL = 5e-3     # bfloat16 outputs: sum|gpu - oracle| / sum|oracle|
MU_MAX_ABS = 1e-5        # updated centroids (float32 state)


def dev_tensor(t, device="cuda"):
    """A synthetic.Tensor (or float32 numpy array) as a device tensor with the
    same bytes."""
    if hasattr(t, "storage") and hasattr(t, "dtype") and t.dtype in ("f32", "bf16"):
        st = t.storage
        if t.dtype == "bf16":
            return torch.from_numpy(st.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(st).to(device)
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)


def host(x: torch.Tensor) -> np.ndarray:
    x = x.detach()
    if x.dtype == torch.bfloat16:
        x = x.float()
    return x.cpu().numpy().astype(np.float64) if x.is_floating_point() else x.cpu().numpy()


def assert_close_out(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "out"):
    """`dtype` is the input dtype of the computation; `got` is its float32 output."""
    err = np.abs(got - want)
    if err.size == 0:
        return
    at = np.unravel_index(np.argmax(err), err.shape)
    where = f"at {tuple(int(i) for i in at)}: got {got[at]:.6g} want {want[at]:.6g}"
    if dtype == "f32":
        assert err.max() <= F32_MAX_ABS, f"{what}: max-abs {err.max():.3e} > {F32_MAX_ABS} {where}"
        return
    denom = np.abs(want).sum()
    mean_rel = err.sum() / denom if denom > 0 else err.sum()
    assert err.max() <= BF16_MAX_ABS, f"{what}: max-abs {err.max():.3e} > {BF16_MAX_ABS} {where}"
    assert mean_rel <= BF16_MEAN_REL, f"{what}: mean-rel {mean_rel:.3e} > {BF16_MEAN_REL}"


def assert_exact_rounding(out_storage: torch.Tensor, out_f32: torch.Tensor):
    """A bf16 output must be exactly the round-to-nearest-even of the float32
    output of the same computation (a float32 one must equal it)."""
    assert out_f32.dtype == torch.float32
    if out_storage.dtype == torch.bfloat16:
        want = out_f32.to(torch.bfloat16)
    else:
        want = out_f32
    eq = torch.eq(out_storage.view(torch.int16) if out_storage.dtype == torch.bfloat16 else out_storage,
                  want.view(torch.int16) if want.dtype == torch.bfloat16 else want)
    assert bool(eq.all()), f"{int((~eq).sum())} elements differ from the rounded float32 output"


def assert_mask_matches(mask: np.ndarray, idx: np.ndarray, n: int):
    """The membership bitmask [B,H,n,KW] must have bit c of token t set exactly
    when t appears in idx[b,h,c]."""
    B, H, k, _ = idx.shape
    KW = (k + 31) // 32
    want = np.zeros((B, H, n, KW), dtype=np.uint32)
    for b in range(B):
        for h in range(H):
            for c in range(k):
                want[b, h, idx[b, h, c], c // 32] |= np.uint32(1 << (c % 32))
    assert np.array_equal(mask.astype(np.int64).astype(np.uint32), want)


def check_membership(orc, gpu_idx, orc_idx, orc_margin, qk_value, mu, w):
    """Equal rows wherever the oracle's margin exceeds MARGIN; elsewhere the GPU
    row must be a valid top-w of the oracle's scores within MARGIN.  Returns
    the boolean [B,H,k] array of clusters whose rows differ."""
    B, H, k, _ = orc_idx.shape
    same = (gpu_idx == orc_idx).all(-1)
    robust = orc_margin > MARGIN
    bad = np.argwhere(robust & ~same)
    assert bad.size == 0, f"membership differs on {len(bad)} clusters with margin > {MARGIN}: {bad[:5]}"
    for b, h, c in np.argwhere(~same):
        row = gpu_idx[b, h, c]
        assert np.all(np.diff(row) > 0) and row.min() >= 0 and row.max() < qk_value.shape[2]
        xhat, _ = orc.normalize(qk_value[b, h])
        s = orc.scores(xhat, mu[h, c:c + 1])[0]
        order = np.sort(s)[::-1]
        sw, sw1 = order[w - 1], (order[w] if w < len(s) else -np.inf)
        chosen = np.zeros(len(s), bool)
        chosen[row] = True
        assert np.all(s[chosen] >= sw - MARGIN) and np.all(s[~chosen] <= sw1 + MARGIN)
    return ~same


def tokens_touched(idx_a, idx_b, differs, n):
    """[B,H,n] mask of tokens that belong, under either membership, to a
    cluster whose rows differ."""
    B, H = idx_a.shape[:2]
    touched = np.zeros((B, H, n), bool)
    for b, h, c in np.argwhere(differs):
        touched[b, h, idx_a[b, h, c]] = True
        touched[b, h, idx_b[b, h, c]] = True
    return touched


def partition_cluster_range(orc, x_bh, mu_h, tie=MARGIN):
    """Per token of one (batch, head), the range [lo, hi] of partition clusters
    its place in the order (nearest centroid, descending score, position)
    allows, given the oracle's float64 scores and that any two keys within
    ``tie`` of each other may be ordered either way by float32 scores.

    A token's label may be any centroid within ``tie`` of its best one.  Token
    u certainly precedes t when every label u may take is below every label t
    may take, or when both have one possible label, the same, and u's score
    exceeds t's by more than ``tie``; certainly follows likewise.  Then t's
    rank lies in [#before, n - 1 - #after] and its cluster in that range
    divided by n/k.  Returns (lo, hi) int arrays [n]."""
    xh, _ = orc.normalize(x_bh)
    s = xh @ mu_h.T                                        # [n, k]
    n, k = s.shape
    w = n // k
    top = s.max(axis=1)
    allowed = s >= top[:, None] - tie
    lab_lo = np.argmax(allowed, axis=1)
    lab_hi = k - 1 - np.argmax(allowed[:, ::-1], axis=1)
    unique = lab_lo == lab_hi
    best = s[np.arange(n), lab_lo]
    before = np.searchsorted(np.sort(lab_hi), lab_lo, side="left")
    after = n - np.searchsorted(np.sort(lab_lo), lab_hi, side="right")
    for c in range(k):
        sel = np.flatnonzero(unique & (lab_lo == c))
        if sel.size == 0:
            continue
        bs = np.sort(best[sel])
        bt = best[sel]
        before[sel] += bs.size - np.searchsorted(bs, bt + tie, side="right")
        after[sel] += np.searchsorted(bs, bt - tie, side="left")
    return before // w, (n - 1 - after) // w


def check_partition(orc, got_idx, x_value, mu, tie=MARGIN):
    """A partition membership [B,H,k,n/k] from the device must hold every token
    once, list rows by ascending position, and put each token in a cluster its
    oracle rank allows (partition_cluster_range).  Returns (tokens whose cluster
    is fixed, tokens with a choice)."""
    B, H, k, w = got_idx.shape
    n = k * w
    pinned = free = 0
    for b in range(B):
        for h in range(H):
            g = got_idx[b, h]
            np.testing.assert_array_equal(np.sort(g.ravel()), np.arange(n))
            assert np.all(np.diff(g, axis=1) > 0), "rows not in ascending position"
            cl = np.empty(n, np.int64)
            cl[g.ravel()] = np.repeat(np.arange(k), w)
            lo, hi = partition_cluster_range(orc, x_value[b, h], mu[h], tie)
            bad = np.flatnonzero((cl < lo) | (cl > hi))
            assert bad.size == 0, (f"(b={b}, h={h}): {bad.size} tokens in a cluster their rank "
                                   f"excludes, e.g. token {bad[0]} in {cl[bad[0]]}, allowed "
                                   f"[{lo[bad[0]]}, {hi[bad[0]]}]")
            pinned += int((lo == hi).sum())
            free += int((lo != hi).sum())
    return pinned, free
