"""HIP-graph replay of the layer step: a captured step must give, on every
replay, bit-identical results to the same step run eagerly (the library
clears its own scratch with kernels, never with memset nodes), with eager
work and synchronisations between the replays."""
import math

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


CASES = {
    "mixed_small": S.Config(70, "mixed_small", "bf16", 2, 2, 2, 1000, 64, 16, 64, 100),
    "long_like_bwd": S.Config(71, "long_like_bwd", "bf16", 1, 2, 1, 2048, 128, 16, 128, 256,
                              backward=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(rt, name):
    cfg = CASES[name]
    inp = S.make_inputs(cfg)
    B, R, n, d, k, w = cfg.B, cfg.R, cfg.n, cfg.d, cfg.k, cfg.w
    scale = 1.0 / math.sqrt(d)
    qk, v = dev_tensor(inp["qk"]), dev_tensor(inp["v"])
    ql, kl, vl = (dev_tensor(inp[x]) for x in ("q_local", "k_local", "v_local"))
    mu0 = dev_tensor(inp["mu"])
    mu = mu0.clone()
    inv = torch.empty((B, R, n), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, R, k, w), dtype=torch.int32, device="cuda")
    mask = torch.empty((B, R, n, rt.mask_words(k)), dtype=torch.int32, device="cuda")
    sum_q = torch.empty((B, R, k, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, R, k, w), dtype=torch.float32, device="cuda")
    out, out_l = torch.empty_like(qk), torch.empty_like(ql)
    grads = tuple(torch.empty((B, R, n, d), dtype=torch.float32, device="cuda") for _ in range(3))
    dout = dev_tensor(S.normal_tensor(1000 * cfg.cfg_id + 3, (B, R, n, d), "bf16"))
    ws = {op: torch.empty(max(1, rt.workspace_bytes(op, B, R, n, d, k, w)), dtype=torch.uint8,
                          device="cuda") for op in ("route", "routed_attn", "routed_attn_bwd")}

    def step():
        rt.route(qk, mu, w, out=(inv, idx, mask), ws=ws["route"])
        rt.routed_attn(qk, qk, v, idx, inv, inv, scale=scale, mask=mask, sums=(sum_q, None),
                       out=out, lse=lse, ws=ws["routed_attn"])
        rt.centroid_update_sums_(mu, sum_q, cfg.lam)
        if cfg.backward:
            rt.routed_attn_bwd(qk, qk, v, idx, lse, dout, inv, inv, scale=scale, out=grads,
                               ws=ws["routed_attn_bwd"])
        rt.local_attn(ql, kl, vl, cfg.window, scale=scale, out=out_l)

    def snapshot():
        return [t.clone() for t in (inv, idx, mask, out, lse, mu, out_l, *grads)]

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
        want = snapshot()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        torch.cuda.synchronize()
        for rep in range(4):
            mu.copy_(mu0)
            for t in (out, out_l, lse, *grads):   # eager work between replays
                t.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = snapshot()
            for i, (g, w_) in enumerate(zip(got, want)):
                if not (cfg.backward or i < 7):
                    continue
                assert torch.equal(g, w_), f"replay {rep}: tensor {i} differs from the eager step"
