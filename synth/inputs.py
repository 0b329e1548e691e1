"""Seeded generators for NVFP4 weights, FP16 activations and top-k routings.

Every generator takes a ``numpy.random.Generator`` (PCG64 seeded from a ``SeedSequence`` of
``[workload_id, weight_set, route_pattern]``), so a case is reproduced from three integers.

Storage formats (the format the library consumes):
  codes   uint8 [G, N, K/2]   two E2M1 codes per byte, the even k in the low nibble
  scales  uint8 [G, N, K/16]  one E4M3FN byte per 16-element K-block
  gscale  float32 [G]         one FP32 global scale per group (expert, or the whole tensor)

The workloads are those of the grouped-MoE and dense-projection kernels described on the
"[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page (section "Latest grouped-MoE screen":
512 experts, top-10, C16 decode; the 8192-token top-10 prefill of the "[Perf][SM70] Optimize
Qwen3.8 Flash Next prefill" page) with synthetic weights, since the real checkpoints are not public.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "SCALE_BYTES_POW2",
    "rng_for",
    "nvfp4_weights",
    "activations",
    "softmax_weights",
    "routing_uniform",
    "routing_zipf",
    "routing_singleton",
    "routing_shared",
    "routing_repeat_invalid",
    "ROUTINGS",
    "MoEShape",
    "TINY",
    "DECODE",
    "PREFILL",
    "DENSE_N",
    "DENSE_K",
    "DENSE_MS",
    "moe_case",
    "dense_case",
    "device_nvfp4_weights",
    "active_experts",
    "router_logits",
    "fp8_channel_weights",
    "shared_expert",
]

# E4M3FN bytes of 2^u for integer u in [-8, -4]: 2^-8 and 2^-7 are E4M3 subnormals (0x02, 0x04),
# 2^-6 .. 2^-4 are normals (0x08, 0x10, 0x18). Listed as bytes; no decoding happens here.
SCALE_BYTES_POW2 = np.array([0x02, 0x04, 0x08, 0x10, 0x18], dtype=np.uint8)


def rng_for(workload: int, weight_set: int = 0, route_pattern: int = 0) -> np.random.Generator:
    """PCG64 generator for one (workload, weight set, route pattern) triple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, weight_set, route_pattern])))


def nvfp4_weights(rng: np.random.Generator, groups: int, rows: int, k: int,
                  scale_bytes: np.ndarray = SCALE_BYTES_POW2, gscale: float = 1.0):
    """Uniform random code bytes (uniform over the 16 codes per nibble), scale bytes drawn uniformly
    from ``scale_bytes``, and a constant global scale. Returns (codes, scales, gscale)."""
    assert k % 16 == 0
    codes = rng.integers(0, 256, size=(groups, rows, k // 2), dtype=np.uint8)
    scales = rng.choice(np.asarray(scale_bytes, dtype=np.uint8), size=(groups, rows, k // 16))
    gs = np.full((groups,), gscale, dtype=np.float32)
    return codes, scales.astype(np.uint8), gs


def activations(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    """N(0,1) samples rounded to float16 (round-to-nearest-even by numpy's cast)."""
    return rng.standard_normal((m, k)).astype(np.float16)


def softmax_weights(rng: np.random.Generator, m: int, topk: int) -> np.ndarray:
    """Top-k combine weights: a softmax over ``topk`` N(0,1) logits per token (the ids are drawn
    uniformly, so they cannot be the logits' own top-k)."""
    z = rng.standard_normal((m, topk))
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def routing_uniform(rng, m, topk, e):
    """Distinct uniform expert ids per token."""
    ids = np.stack([rng.choice(e, size=topk, replace=False) for _ in range(m)]) if m else np.zeros((0, topk))
    return ids.astype(np.int32).reshape(m, topk)


def routing_zipf(rng, m, topk, e, s=1.2):
    """Zipf(s) popularity over a seeded permutation of the experts; each token draws ``topk``
    distinct experts without replacement (Gumbel-top-k over log-popularity)."""
    perm = rng.permutation(e)
    logp = -s * np.log(np.arange(1, e + 1, dtype=np.float64))
    ids = np.zeros((m, topk), dtype=np.int32)
    for t in range(m):
        g = logp + rng.gumbel(size=e)
        ids[t] = perm[np.argsort(-g, kind="stable")[:topk]]
    return ids


def routing_singleton(rng, m, topk, e):
    """All m*topk pairs get distinct experts (needs m*topk <= e)."""
    assert m * topk <= e
    return rng.permutation(e)[: m * topk].astype(np.int32).reshape(m, topk)


def routing_shared(rng, m, topk, e):
    """Every token uses the same ``topk`` experts in the same slot order."""
    row = rng.choice(e, size=topk, replace=False).astype(np.int32)
    return np.tile(row, (m, 1)).reshape(m, topk)


def routing_repeat_invalid(rng, m, topk, e):
    """Distinct ids, then slot (t mod topk) := -1 and slot ((t+3) mod topk) := the id in slot
    ((t+5) mod topk); when m >= 2 the last token is all -1."""
    ids = routing_uniform(rng, m, topk, e)
    for t in range(m):
        ids[t, (t + 3) % topk] = ids[t, (t + 5) % topk]
        ids[t, t % topk] = -1
    if m >= 2:
        ids[m - 1, :] = -1
    return ids


ROUTINGS = {
    "uniform": routing_uniform,
    "zipf": routing_zipf,
    "singleton": routing_singleton,
    "shared": routing_shared,
    "repeat_invalid": routing_repeat_invalid,
}


@dataclass(frozen=True)
class MoEShape:
    m: int
    e: int
    topk: int
    k: int  # hidden size (W13 reduction length, W2 output rows)
    i: int  # expert intermediate size

    @property
    def pairs(self) -> int:
        return self.m * self.topk


# Tiny grouped MoE: 1 token, 8 experts, top-2, K=256, I=128.
TINY = MoEShape(m=1, e=8, topk=2, k=256, i=128)
# One rank's share of the C16 grouped decode: 16 tokens, 512 experts, top-10, K=2048, I=512.
DECODE = MoEShape(m=16, e=512, topk=10, k=2048, i=512)
# Prefill-size grouped MoE: 8192 tokens, otherwise as DECODE.
PREFILL = MoEShape(m=8192, e=512, topk=10, k=2048, i=512)
# Dense QPN-style projection: W [4352, 5120], M in {1, 2, 4, 8, 16, 32}.
DENSE_N, DENSE_K = 4352, 5120
DENSE_MS = (1, 2, 4, 8, 16, 32)

WORKLOAD_IDS = {"tiny": 0, "dense": 1, "decode": 2, "stress": 3, "prefill": 4, "route": 5}


def moe_case(shape: MoEShape, routing: str = "uniform", weight_set: int = 0, route_pattern: int = 0,
             workload: str = "decode", gscale13: float = 1.0, gscale2: float = 1.0,
             scale_bytes: np.ndarray = SCALE_BYTES_POW2, weights=None):
    """One grouped-MoE input set. Weights depend on (workload, weight_set) only, routing and
    activations on (workload, weight_set, route_pattern), so several route patterns share weights."""
    wid = WORKLOAD_IDS[workload]
    if weights is None:
        rw = rng_for(wid, weight_set, 0)
        w13 = nvfp4_weights(rw, shape.e, 2 * shape.i, shape.k, scale_bytes, gscale13)
        w2 = nvfp4_weights(rw, shape.e, shape.k, shape.i, scale_bytes, gscale2)
        weights = (w13, w2)
    rr = rng_for(wid, weight_set, 1000 + route_pattern)
    x = activations(rr, shape.m, shape.k)
    ids = ROUTINGS[routing](rr, shape.m, shape.topk, shape.e)
    tw = softmax_weights(rr, shape.m, shape.topk)
    return {"shape": shape, "x": x, "ids": ids, "topk_weights": tw, "w13": weights[0], "w2": weights[1]}


def dense_case(m: int, n: int = DENSE_N, k: int = DENSE_K, weight_set: int = 0, gscale: float = 1.0,
               scale_bytes: np.ndarray = SCALE_BYTES_POW2):
    rw = rng_for(WORKLOAD_IDS["dense"], weight_set, 0)
    w = nvfp4_weights(rw, 1, n, k, scale_bytes, gscale)
    rx = rng_for(WORKLOAD_IDS["dense"], weight_set, 1000 + m)
    return {"x": activations(rx, m, k), "w": w}


def device_nvfp4_weights(seed: int, groups: int, rows: int, k: int, device="cuda",
                         scale_bytes: np.ndarray = SCALE_BYTES_POW2, gscale: float = 1.0):
    """Bulk random NVFP4 storage drawn on the device with a seeded torch generator (for benchmark
    weight sets, which are too large to draw on the host): uniform code bytes, scale bytes drawn
    uniformly from ``scale_bytes``, constant global scale. Returns (codes, scales, gscale) tensors."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    codes = torch.randint(0, 256, (groups, rows, k // 2), dtype=torch.uint8, generator=g, device=device)
    table = torch.as_tensor(np.asarray(scale_bytes, dtype=np.uint8), device=device)
    idx = torch.randint(0, len(scale_bytes), (groups, rows, k // 16), generator=g, device=device)
    scales = table[idx].contiguous()
    gs = torch.full((groups,), gscale, dtype=torch.float32, device=device)
    return codes, scales, gs


def active_experts(ids: np.ndarray, e: int) -> int:
    """Number of distinct valid expert ids in a routing (the experts whose weights a grouped layer reads)."""
    v = ids[(ids >= 0) & (ids < e)]
    return int(np.unique(v).size)


def router_logits(rng: np.random.Generator, m: int, e: int, kind: str = "normal") -> np.ndarray:
    """Router logits float32 [m, e].
      normal   N(0,1)
      ties     integers in [-2, 2], each zero given a random sign (many equal values, +0 and -0)
      special  N(0,1) with about 2% NaN, 2% +inf, 2% -inf and 2% signed zeros per row"""
    if kind == "normal":
        return rng.standard_normal((m, e)).astype(np.float32)
    if kind == "ties":
        x = rng.integers(-2, 3, size=(m, e)).astype(np.float32)
        neg = rng.random((m, e)) < 0.5
        x[(x == 0) & neg] = np.float32(-0.0)
        return x
    if kind == "special":
        x = rng.standard_normal((m, e)).astype(np.float32)
        u = rng.random((m, e))
        x[u < 0.02] = np.nan
        x[(u >= 0.02) & (u < 0.04)] = np.inf
        x[(u >= 0.04) & (u < 0.06)] = -np.inf
        x[(u >= 0.06) & (u < 0.07)] = np.float32(0.0)
        x[(u >= 0.07) & (u < 0.08)] = np.float32(-0.0)
        return x
    raise ValueError(kind)


def fp8_channel_weights(rng: np.random.Generator, rows: int, k: int):
    """Channel-FP8 weights: uniform random E4M3FN bytes (every exponent, subnormals and both zeros
    included) with the NaN patterns 0x7F/0xFF replaced by 0x7E/0xFE, and one float32 scale per row
    2^u, u uniform in [-6, -4]. Returns (codes uint8 [rows, k], scale float32 [rows])."""
    codes = rng.integers(0, 256, size=(rows, k), dtype=np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    scale = np.exp2(rng.uniform(-6.0, -4.0, size=rows)).astype(np.float32)
    return codes, scale


def shared_expert(rng: np.random.Generator, k: int, i: int, gscale: float = 1.0):
    """A shared expert for a MoE layer of hidden size k: NVFP4 gate/up weights [2i, k], down weights
    [k, i], and the fp16 shared-gate vector g [k] drawn N(0, 1/k) (so x . g is about N(0, 1))."""
    w13 = nvfp4_weights(rng, 1, 2 * i, k, gscale=gscale)
    w2 = nvfp4_weights(rng, 1, k, i, gscale=gscale)
    g = (rng.standard_normal(k) / np.sqrt(k)).astype(np.float16)
    return {"w13": w13, "w2": w2, "g": g, "layout": 0}
