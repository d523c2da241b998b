"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module draws random numbers and rounds them to the storage precision;
it holds none of the routed-attention arithmetic.  Both sides of every parity
check receive exactly the bytes produced here.

Generator: SplitMix64 used as a counter-based stream (output i of stream
``seed`` is ``mix64(seed + (i + 1) * 0x9E3779B97F4A7C15)``, the published
SplitMix64 definition of Steele, Lea and Flood, OOPSLA 2014), turned into
standard normals by the Box-Muller transform, then rounded float64 -> float32
(round to nearest even) and, for bf16 tensors, float32 -> bfloat16 (round to
nearest even on the bit pattern).

Seeds: ``1000 * config_id + tensor_id`` with tensor ids qk 0, v 1, mu 2,
dO 3, local q 4, local k 5, local v 6, skew centres 7, skew positions 8,
skew noise 9, per-layer weights 100 + 8*layer + j.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_IDS = {
    "qk": 0, "v": 1, "mu": 2, "dout": 3, "q_local": 4, "k_local": 5,
    "v_local": 6, "skew_centres": 7, "skew_pos": 8, "skew_noise": 9,
}


def splitmix64(seed: int, count: int, offset: int = 0) -> np.ndarray:
    """Outputs ``offset .. offset+count-1`` of the SplitMix64 stream ``seed``."""
    i = np.arange(offset + 1, offset + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, count: int) -> np.ndarray:
    """Doubles in (0, 1]: the top 53 bits of each SplitMix64 output, plus one ulp."""
    z = splitmix64(seed, count)
    return ((z >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normal(seed: int, shape) -> np.ndarray:
    """Standard normals (float64) by Box-Muller over consecutive uniform pairs."""
    count = int(np.prod(shape)) if len(shape) else 1
    pairs = (count + 1) // 2
    u = uniform01(seed, 2 * pairs)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * pairs, dtype=np.float64)
    z[0::2] = r * np.cos(2.0 * math.pi * u2)
    z[1::2] = r * np.sin(2.0 * math.pi * u2)
    return z[:count].reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Tensor:
    """One synthetic tensor: its exact value (float64) and its storage bytes."""
    value: np.ndarray          # float64, exactly the stored value
    dtype: str                 # "f32" or "bf16"

    @property
    def storage(self) -> np.ndarray:
        """The array whose bytes go to the device (float32 or uint16 bits)."""
        if self.dtype == "f32":
            return self.value.astype(np.float32)
        return f32_to_bf16_bits(self.value.astype(np.float32))


def rounded(x: np.ndarray, dtype: str) -> Tensor:
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return Tensor(x32.astype(np.float64), "f32")
    if dtype == "bf16":
        return Tensor(bf16_bits_to_f64(f32_to_bf16_bits(x32)), "bf16")
    raise ValueError(dtype)


def normal_tensor(seed: int, shape, dtype: str, sigma: float = 1.0) -> Tensor:
    return rounded(sigma * normal(seed, shape), dtype)


def unit_rows_f32(seed: int, rows: int, d: int) -> np.ndarray:
    """``rows`` random unit vectors in R^d (Gaussian draw scaled to length 1),
    stored as float32; returned as the float64 value of the float32s."""
    g = normal(seed, (rows, d))
    g = g / np.sqrt((g * g).sum(axis=1, keepdims=True))
    return g.astype(np.float32).astype(np.float64)


def skewed_qk(cfg_id: int, shape, dtype: str, frac: float = 0.10,
              n_centres: int = 8, sigma: float = 0.05) -> Tensor:
    """N(0,1) tokens, except ``frac`` of the sequence positions (drawn uniformly
    without replacement, per batch row and head) which are replaced by
    centre_j + sigma*N(0, I_d), j drawn uniformly from ``n_centres`` centres
    ~ N(0, I_d) (one set of centres per head)."""
    B, H, n, d = shape
    base = normal(1000 * cfg_id + TENSOR_IDS["qk"], shape)
    centres = normal(1000 * cfg_id + TENSOR_IDS["skew_centres"], (H, n_centres, d))
    m = int(round(frac * n))
    keys = splitmix64(1000 * cfg_id + TENSOR_IDS["skew_pos"], B * H * n).reshape(B, H, n)
    pick = splitmix64(1000 * cfg_id + TENSOR_IDS["skew_pos"], B * H * m,
                      offset=B * H * n).reshape(B, H, m)
    noise = normal(1000 * cfg_id + TENSOR_IDS["skew_noise"], (B, H, m, d))
    for b in range(B):
        for h in range(H):
            pos = np.argsort(keys[b, h], kind="stable")[:m]
            j = (pick[b, h] % np.uint64(n_centres)).astype(np.int64)
            base[b, h, pos] = centres[h, j] + sigma * noise[b, h]
    return rounded(base, dtype)


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload of the routed-attention layer."""
    cfg_id: int
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    R: int              # routed heads
    L: int              # local (sliding-window) heads
    n: int
    d: int
    k: int
    w: int
    window: int         # local window (0: no local heads)
    lam: float = 0.999
    causal: bool = True
    skew: bool = False
    backward: bool = False

    @property
    def tokens(self) -> int:
        return self.B * self.n

    def scaled(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": Config(1, "tiny", "f32", 1, 1, 0, 64, 16, 4, 16, 0),
    "routed": Config(2, "routed", "bf16", 4, 8, 0, 1024, 64, 32, 32, 0),
    "mixed": Config(3, "mixed", "bf16", 2, 8, 8, 4096, 64, 64, 64, 256),
    "long": Config(4, "long", "bf16", 1, 8, 4, 8192, 128, 64, 128, 512),
    "stress": Config(5, "stress", "bf16", 1, 8, 8, 32768, 64, 128, 256, 256,
                     skew=True, backward=True),
}


def make_inputs(cfg: Config) -> dict:
    """All tensors of one workload, seeded by ``1000*cfg_id + tensor_id``."""
    s = 1000 * cfg.cfg_id
    shape_r = (cfg.B, cfg.R, cfg.n, cfg.d)
    out = {}
    if cfg.skew:
        out["qk"] = skewed_qk(cfg.cfg_id, shape_r, cfg.dtype)
    else:
        out["qk"] = normal_tensor(s + TENSOR_IDS["qk"], shape_r, cfg.dtype)
    out["v"] = normal_tensor(s + TENSOR_IDS["v"], shape_r, cfg.dtype)
    mu = unit_rows_f32(s + TENSOR_IDS["mu"], cfg.R * cfg.k, cfg.d)
    out["mu"] = mu.reshape(cfg.R, cfg.k, cfg.d)
    if cfg.L > 0:
        shape_l = (cfg.B, cfg.L, cfg.n, cfg.d)
        for name in ("q_local", "k_local", "v_local"):
            out[name] = normal_tensor(s + TENSOR_IDS[name], shape_l, cfg.dtype)
    if cfg.backward:
        out["dout"] = normal_tensor(s + TENSOR_IDS["dout"], shape_r, cfg.dtype)
    return out


# ---- the layer stack of the long workload ---------------------------------------------
# x ~ N(0, 1) [B, n, d_model]; per layer l: W_in [(2R+3L)d, d_model] and W_o
# [d_model, (R+L)d] ~ N(0, 1/fan_in), centroids as in make_inputs.  Seeds:
# 1000*cfg_id + 10 for x, 1000*cfg_id + 100 + 8l + j for layer l (j = 0 W_in,
# 1 W_o, 2 centroids).

@dataclasses.dataclass(frozen=True)
class StackConfig:
    cfg_id: int
    name: str
    B: int
    n: int
    dm: int             # model width
    d: int              # head width
    R: int              # routed heads per layer
    L: int              # local heads per layer
    k: int
    w: int
    window: int
    layers: int
    lam: float = 0.999

    def scaled(self, **kw) -> "StackConfig":
        return dataclasses.replace(self, **kw)


def stack_x(sc: StackConfig) -> Tensor:
    return normal_tensor(1000 * sc.cfg_id + 10, (sc.B, sc.n, sc.dm), "bf16")


def stack_layer(sc: StackConfig, layer: int) -> dict:
    s = 1000 * sc.cfg_id + 100 + 8 * layer
    n_in = (2 * sc.R + 3 * sc.L) * sc.d
    n_heads = (sc.R + sc.L) * sc.d
    return {
        "w_in": normal_tensor(s, (n_in, sc.dm), "bf16", sigma=1.0 / np.sqrt(sc.dm)),
        "w_o": normal_tensor(s + 1, (sc.dm, n_heads), "bf16", sigma=1.0 / np.sqrt(n_heads)),
        "mu": unit_rows_f32(s + 2, sc.R * sc.k, sc.d).reshape(sc.R, sc.k, sc.d),
    }


STACKS = {
    # the long-sequence layer (8 routed + 4 local heads of width 128, k = 64,
    # w = 128, window 512) at model width 1024, 22 layers
    "long_stack": StackConfig(4, "long_stack", 1, 8192, 1024, 128, 8, 4, 64, 128, 512, 22),
}


def separated_tokens(seed: int, B: int, H: int, n: int, d: int, k: int, dtype: str = "bf16",
                     spacing: float = 1.5e-3, weights=None):
    """Tokens gathered around k random unit centres, for inputs whose
    nearest-centre assignment and within-group order hold no near-equal
    values.  Returns (tokens [B,H,n,d] as a Tensor, centres [H,k,d] float32
    values).

    Each token draws its group c with probability proportional to a weight in
    [0.7, 1.3] per (head, group) (or to `weights` [k], the same for every head),
    so groups are unequal in size.  The j-th token of a group (in a seeded
    random order) is 2 * (cos(a) m_c + sin(a) u), with
    cos(a) = 0.995 - spacing * j and u a random unit vector orthogonal to the
    centre m_c, so the cosines inside a group are `spacing` apart (a group must
    hold fewer than 0.4 / spacing tokens for them to stay nearest their own
    centre)."""
    mu = unit_rows_f32(seed, H * k, d).reshape(H, k, d)
    weight = 0.7 + 0.6 * uniform01(seed + 1, H * k).reshape(H, k)
    if weights is not None:
        weight = np.broadcast_to(np.asarray(weights, dtype=np.float64), (H, k))
    u_lab = uniform01(seed + 2, B * H * n).reshape(B, H, n)
    order_keys = splitmix64(seed + 3, B * H * n).reshape(B, H, n)
    g = normal(seed + 4, (B, H, n, d))
    x = np.empty((B, H, n, d))
    for b in range(B):
        for h in range(H):
            cdf = np.cumsum(weight[h]) / weight[h].sum()
            lab = np.minimum(np.searchsorted(cdf, u_lab[b, h], side="left"), k - 1)
            cos_a = np.empty(n)
            for c in range(k):
                sel = np.flatnonzero(lab == c)
                rank = np.argsort(np.argsort(order_keys[b, h, sel], kind="stable"), kind="stable")
                cos_a[sel] = 0.995 - spacing * rank
            m = mu[h, lab]                                        # [n, d]
            u = g[b, h] - (g[b, h] * m).sum(axis=1, keepdims=True) * m
            u /= np.sqrt((u * u).sum(axis=1, keepdims=True))
            x[b, h] = 2.0 * (cos_a[:, None] * m + np.sqrt(1.0 - cos_a[:, None] ** 2) * u)
    return rounded(x, dtype), mu
