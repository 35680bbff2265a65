"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the attention method: it only draws
tensors.  Values are N(0, 1) from a CPU ``torch.Generator`` (seed 42 is the
training seed of the page-1 recipe), drawn as float32 and rounded to bfloat16
(round to nearest even) where the workload says bf16.  Both the HIP path and
the oracle receive identical values (the oracle widens them exactly to fp64).

Workload shapes follow the pages: the page-1 model layer (8 query heads over
2 key/value heads, head dim 64, sequence 1024, 32,768 tokens per batch) and
the page-3 context length 2048.
"""

import torch

SEED = 42

# name -> shape description (no method arithmetic; consumers derive offsets).
WORKLOADS = {
    "tiny_fp32": dict(batch=1, seqlen=64, hq=1, hkv=1, head_dim=16,
                      dtype="f32", window=4, alpha=0.75, rope_theta=1e4),
    "page1_fixed": dict(batch=32, seqlen=1024, hq=8, hkv=2, head_dim=64,
                        dtype="bf16", window=8, alpha=1.0, rope_theta=1e4),
    "page1_staggered": dict(batch=32, seqlen=1024, hq=8, hkv=2, head_dim=64,
                            dtype="bf16", windows=(6, 8, 10, 12), layers=16,
                            stride=7, rope_theta=1e4),
    "page1_learned_step": dict(batch=32, seqlen=1024, hq=8, hkv=2, head_dim=64,
                               dtype="bf16", window=10, rope_theta=1e4),
    "ctx2048_christoffel": dict(batch=8, seqlen=2048, hq=4, hkv=4, head_dim=64,
                                dtype="bf16", m=128, k=1024, rope_theta=0.0),
    "ctx2048_powerlaw": dict(batch=8, seqlen=2048, hq=4, hkv=4, head_dim=64,
                             dtype="bf16", radius=8, sigma=0.8, draws=47,
                             width=64, rope_theta=0.0),
}


def _torch_dtype(dtype):
    if dtype in ("f32", torch.float32):
        return torch.float32
    if dtype in ("bf16", torch.bfloat16):
        return torch.bfloat16
    raise ValueError("dtype must be f32 or bf16")


def randn(shape, seed, dtype="f32"):
    """N(0,1) CPU tensor of `shape`, drawn in fp32 then rounded to `dtype`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return x.to(_torch_dtype(dtype))


def uniform(seed):
    """One U(0,1) float64 drawn from its own generator."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return float(torch.rand((1,), generator=g, dtype=torch.float64).item())


def qkv(batch, seqlen, hq, hkv, head_dim, dtype="f32", seed=SEED):
    """Q [B,n,Hq,D], K and V [B,n,Hkv,D], drawn in that order (seed, +1, +2)."""
    q = randn((batch, seqlen, hq, head_dim), seed, dtype)
    k = randn((batch, seqlen, hkv, head_dim), seed + 1, dtype)
    v = randn((batch, seqlen, hkv, head_dim), seed + 2, dtype)
    return q, k, v


def upstream(batch, seqlen, hq, head_dim, dtype="f32", seed=SEED):
    """Upstream gradient dO [B,n,Hq,D] (seed + 3)."""
    return randn((batch, seqlen, hq, head_dim), seed + 3, dtype)


def learned_alpha(seed=SEED):
    """A seeded alpha in (0.5, 1.5): 0.5 + U(0,1) from seed + 4."""
    u = uniform(seed + 4)
    u = min(max(u, 1e-6), 1.0 - 1e-6)
    return 0.5 + u


def to_f64(t):
    """Exact widening of a CPU tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
