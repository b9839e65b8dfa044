"""Seeded random tensors. Layout everywhere: [batch, heads, tokens, head_dim], frame-major tokens."""
import math

import torch


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal_qkv(batch, heads, N, d, seed=0, dtype=torch.bfloat16):
    """Q, K, V ~ N(0, 1) drawn in float32 on the CPU, then cast to ``dtype``."""
    g = _gen(seed)
    q = torch.randn(batch, heads, N, d, generator=g, dtype=torch.float32)
    k = torch.randn(batch, heads, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(batch, heads, N, d, generator=g, dtype=torch.float32)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def planted_qkv(batch, F, H, W, d, kinds, seed=0, strength=0.8, dtype=torch.bfloat16):
    """Q, K, V with unit-variance entries and a planted head structure.

    For a head of kind 0, queries and keys of one frame share a random vector;
    for kind 1, queries and keys of one spatial position (same h, w) share one
    across all frames. Each entry is sqrt(strength) * shared + sqrt(1 - strength)
    * noise, so every entry is still N(0, 1). V is plain N(0, 1).
    """
    g = _gen(seed)
    S = H * W
    heads = len(kinds)
    a = math.sqrt(strength)
    c = math.sqrt(1.0 - strength)
    q = torch.randn(batch, heads, F, S, d, generator=g) * c
    k = torch.randn(batch, heads, F, S, d, generator=g) * c
    for h, kind in enumerate(kinds):
        if kind == 0:
            u = torch.randn(batch, F, 1, d, generator=g) * a
        else:
            u = torch.randn(batch, 1, S, d, generator=g) * a
        q[:, h] += u
        k[:, h] += u
    v = torch.randn(batch, heads, F * S, d, generator=g)
    q = q.reshape(batch, heads, F * S, d)
    k = k.reshape(batch, heads, F * S, d)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def census_qkv(batch, heads, N, d, key_class=None, dtype=torch.bfloat16):
    """Q = K = 0 (uniform weights over each row's kept keys) and V[h, k, c] = 1 iff
    key_class[h, k] mod d == c. ``key_class`` is an integer array [heads, N] chosen by the
    caller (default: the key index k itself)."""
    q = torch.zeros(batch, heads, N, d, dtype=dtype)
    k = torch.zeros(batch, heads, N, d, dtype=dtype)
    v = torch.zeros(batch, heads, N, d, dtype=torch.float32)
    idx = torch.arange(N)
    if key_class is None:
        key_class = idx.expand(heads, N)
    key_class = torch.as_tensor(key_class, dtype=torch.int64)
    for h in range(heads):
        v[:, h, idx, key_class[h] % d] = 1.0
    return q, k, v.to(dtype)


def sample_indices(N, n, seed=0):
    """n distinct query ids in [0, N), sorted, as int32."""
    g = _gen(seed)
    return torch.sort(torch.randperm(N, generator=g)[:n]).values.to(torch.int32)
