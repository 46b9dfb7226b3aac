"""Brute-force float64 HSTU layer stack: users padded to the longest sequence,
a dense [B, L, L] visibility mask, full recompute only.

TEST INFRASTRUCTURE ONLY.  It is written as whole-array numpy algebra,
independently of the loop-form oracle in hstu_oracle.c, so the two pin each
other on small inputs.  The bucket here uses the floating formula
floor(4 * log2(1 + delta)); the oracle evaluates it exactly in integers.
"""
from __future__ import annotations

from typing import List

import numpy as np


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _ln(x, eps):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def bucket_float(delta: np.ndarray, num_buckets: int) -> np.ndarray:
    b = np.floor(4.0 * np.log2(1.0 + np.maximum(delta, 0).astype(np.float64)))
    return np.minimum(b, num_buckets - 1).astype(np.int64)


def mask(lengths, n_targets, L: int) -> np.ndarray:
    """[B, L, L] bool: key j visible to query i."""
    B = len(lengths)
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    m = np.zeros((B, L, L), dtype=bool)
    for b in range(B):
        hist = lengths[b] - n_targets[b]
        valid = (i < lengths[b]) & (j < lengths[b])
        m[b] = valid & ((j == i) | ((j < i) & (j < hist)))
    return m


def layer(x_pad, lengths, n_targets, norm_n, w1, w2, rab, num_heads, head_dim, eps=1e-5):
    """x_pad [B, L, d] -> dict of float64 [B, L, ...] (rows past a user's length are junk)."""
    x = np.asarray(x_pad, dtype=np.float64)
    B, L, d = x.shape
    inner = num_heads * head_dim
    xh = _ln(x, eps)
    s = _silu(xh @ np.asarray(w1, np.float64))
    U, V, Q, K = (s[..., c * inner:(c + 1) * inner] for c in range(4))

    def heads(t):
        return t.reshape(B, L, num_heads, head_dim).transpose(0, 2, 1, 3)

    q, k, v = heads(Q), heads(K), heads(V)
    scores = q @ k.transpose(0, 1, 3, 2)                       # [B, H, L, L]
    delta = np.arange(L)[:, None] - np.arange(L)[None, :]
    bias = np.asarray(rab, np.float64)[bucket_float(delta, len(rab))]
    m = mask(lengths, n_targets, L)[:, None, :, :]
    a = np.where(m, _silu(scores + bias[None, None]), 0.0)
    a = a / np.asarray(norm_n, np.float64)[:, None, None, None]
    o = (a @ v).transpose(0, 2, 1, 3).reshape(B, L, inner)
    g = _ln(o, eps) * U
    y = x + g @ np.asarray(w2, np.float64)
    return {"xhat": xh, "u": U, "v": V, "q": Q, "k": K, "o": o, "g": g, "y": y}


def stack(layers, x_users: List[np.ndarray], n_targets, norm_n, num_heads, head_dim, eps=1e-5,
          return_all=False):
    """Full recompute of every position of every user through the stack."""
    lengths = [len(xu) for xu in x_users]
    L = max(lengths) if lengths else 0
    d = x_users[0].shape[1]
    x = np.zeros((len(x_users), L, d))
    for b, xu in enumerate(x_users):
        x[b, :len(xu)] = xu
    outs = []
    for lw in layers:
        out = layer(x, lengths, n_targets, norm_n, lw.w1, lw.w2, lw.rab, num_heads, head_dim, eps)
        outs.append(out)
        x = out["y"]
    ys = [x[b, :lengths[b]] for b in range(len(x_users))]
    return (ys, outs) if return_all else ys
