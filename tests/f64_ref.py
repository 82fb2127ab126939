"""Float64 references used to pin the oracle (no bf16 rounding anywhere).

These are the exact mathematical definitions the oracle rounds its way
through, written with library routines where one exists:

* RMSNorm with (1+w) in float64;
* RoPE as a complex rotation by the exact angle ``p * theta**(-2j/R)`` of the
  pair (x[j], x[j+R/2]) -- computed here from the angle, not from the table;
* attention as ``torch.nn.functional.scaled_dot_product_attention`` in
  float64 on the CPU, with its own GQA head mapping (``enable_gqa``);
* the sigmoid in float64.
"""

from __future__ import annotations

import numpy as np
import torch

U = 2.0 ** -8          # unit roundoff of bf16 (8 significand bits), round to nearest


def bf(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rmsnorm_f64(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * (1.0 + np.asarray(w, np.float64))


def rope_f64(x: np.ndarray, pos, rotary_dim: int = 64, theta: float = 1e7) -> np.ndarray:
    """Rotates pairs (j, j+R/2) of the last axis by angle pos * theta**(-2j/R)."""
    x = np.array(x, np.float64, copy=True)
    half = rotary_dim // 2
    j = np.arange(half, dtype=np.float64)
    ang = np.asarray(pos, np.float64)[..., None] * theta ** (-2.0 * j / rotary_dim)
    z = (x[..., :half] + 1j * x[..., half:rotary_dim]) * np.exp(1j * ang)
    x[..., :half] = z.real
    x[..., half:rotary_dim] = z.imag
    return x


def sdpa_f64(qp: np.ndarray, kp: np.ndarray, v: np.ndarray, q_base: int, mask=None,
             scale: float = 1.0 / 16.0, causal: bool = True) -> np.ndarray:
    """Exact attention of prepared queries/keys.

    qp [rows][Hq][D], kp [Hkv][T][D], v [T][Hkv][D] (float64 values);
    returns ctx [rows][Hq][D].  Visibility is causal on absolute positions
    (every key when ``causal`` is False), ANDed with ``mask`` [rows][T] when given.
    """
    rows, Hq, D = qp.shape
    Hkv, T, _ = kp.shape
    q = torch.from_numpy(np.ascontiguousarray(qp.transpose(1, 0, 2)))[None]       # [1,Hq,rows,D]
    k = torch.from_numpy(np.ascontiguousarray(kp))[None]                          # [1,Hkv,T,D]
    vv = torch.from_numpy(np.ascontiguousarray(np.asarray(v, np.float64).transpose(1, 0, 2)))[None]
    pos = q_base + np.arange(rows)
    vis = np.arange(T)[None, :] <= pos[:, None]
    if not causal:
        vis = np.ones((rows, T), bool)
    if mask is not None:
        vis &= np.asarray(mask) != 0
    m = torch.from_numpy(vis)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, vv, attn_mask=m, scale=scale,
                                                         enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)


def score_max_f64(qp, kp, q_base, mask=None, scale=1.0 / 16.0, causal=True) -> np.ndarray:
    """max_j |s_j| over visible keys, per (row, q head): [rows][Hq]."""
    rows, Hq, D = qp.shape
    Hkv, T, _ = kp.shape
    G = Hq // Hkv
    kk = np.repeat(kp, G, axis=0)                                   # [Hq][T][D]
    s = np.einsum("rhd,htd->rht", qp, kk) * scale
    pos = q_base + np.arange(rows)
    vis = np.arange(T)[None, :] <= pos[:, None]
    if not causal:
        vis = np.ones((rows, T), bool)
    if mask is not None:
        vis &= np.asarray(mask) != 0
    s = np.where(vis[:, None, :], np.abs(s), 0.0)
    return s.max(axis=-1)


def sigmoid_f64(g: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(g, np.float64)))


def torch_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 value (as float64) via torch's round-to-nearest-even cast.

    Goes through float32 only when the value is exact in float32, which holds
    for the products of two bf16 values this is used on.
    """
    t = torch.from_numpy(np.asarray(x, np.float64))
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
