"""rt_route_noalloc (the routing entry point whose score matrix lives in the
library's static per-GPU array) against rt_route (workspace from the caller):
the same kernels, so inverse norms, memberships, membership bits and
normalised rows must be bit-identical, on two calls in a row with the second
smaller than the first (the array keeps the first call's scores; every score
the second call reads is its own)."""
import sys

import numpy as np
import pytest
import torch

import synthetic as S
from _util import dev_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import content_sparse_attention_unit_amd as m
    m._load()
    return m


def _case(rt, B, H, n, d, k, w, seed):
    print(f"[case] route_noalloc B={B} H={H} n={n} d={d} k={k} w={w}", flush=True)
    sys.stdout.flush()
    qk = dev_tensor(S.normal_tensor(seed, (B, H, n, d), "bf16"))
    mu = torch.from_numpy(S.unit_rows_f32(seed + 1, H * k, d).reshape(H, k, d).astype(np.float32)).cuda()
    inv_a, idx_a, mask_a, hat_a = rt.route(qk, mu, w, want_mask=True, want_qk_hat=True)
    out = (torch.empty_like(inv_a), torch.empty_like(idx_a), torch.empty_like(mask_a))
    hat_b = torch.empty_like(hat_a)
    rt.route_noalloc(qk, mu, w, out, qk_hat=hat_b)
    torch.cuda.synchronize()
    assert torch.equal(out[0], inv_a)
    assert torch.equal(out[1], idx_a)
    assert torch.equal(out[2], mask_a)
    assert torch.equal(hat_b, hat_a)


def test_route_noalloc_matches_route_twice(rt):
    _case(rt, 1, 8, 8192, 128, 64, 128, 98_000)       # the long workload's routed heads
    _case(rt, 2, 3, 1000, 64, 10, 77, 98_010)         # smaller, ragged


def test_route_noalloc_rejects_oversize(rt):
    B, H, n, d, k, w = 1, 8, 32768, 64, 128, 256      # 33.5 M scores
    assert B * H * k * n > rt.ROUTE_NOALLOC_MAX_SCORES
    qk = torch.zeros((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    mu = torch.zeros((H, k, d), dtype=torch.float32, device="cuda")
    out = (torch.empty((B, H, n), dtype=torch.float32, device="cuda"),
           torch.full((B, H, k, w), -7, dtype=torch.int32, device="cuda"))
    with pytest.raises(rt.RTError, match="static scratch"):
        rt.route_noalloc(qk, mu, w, out)
    torch.cuda.synchronize()
    assert bool((out[1] == -7).all())                 # nothing was launched
