"""Seeded synthetic inputs for gated GQA causal attention prefill.

This module is the one piece shared by the oracle side and the HIP side: it
draws inputs and holds none of the method's arithmetic (no norm, no RoPE, no
score, softmax or gate).  Everything is counter-based, so any slice of any
tensor can be regenerated without drawing the rest:

* Uniform bits: SplitMix64 (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014).  Output number ``n`` of the
  stream of tensor ``t`` under seed ``s`` is ``mix(s + (t * 2**40 + n + 1) *
  GOLDEN)``, i.e. the (t*2**40+n)-th draw of the generator seeded with ``s``.
* Normals: Box-Muller (Box and Muller, 1958) on consecutive pairs of draws,
  computed in float64, scaled by sigma, cast to float32 and rounded to bf16
  with round-to-nearest-even.
* Visibility mask: row ``i`` sees key ``i`` plus ``budget - 1`` distinct keys
  chosen uniformly without replacement from ``[0, i)`` (all earlier keys when
  ``i < budget``).  The choice takes the ``budget - 1`` smallest random sort
  keys among the earlier positions; the low 13 bits of each sort key hold the
  key index, so there are no ties.
* cos/sin table: ``[n_pos][rotary_dim / 2]`` float32, angle
  ``p * theta ** (-2 j / rotary_dim)`` evaluated in float64 and rounded once
  (the QSA kernel page, "Code review" fixes, F4: the table is built on the
  host in double precision and rounded once; no trig on the device).

bf16 tensors are returned as ``numpy.uint16`` bit patterns.
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_STREAM_STRIDE = 1 << 40

# Stream ids, one per drawn tensor (the draw order of the workload recipe).
STREAM_QG_Q = 0
STREAM_QG_GATE = 1
STREAM_K = 2
STREAM_V = 3
STREAM_WQ = 4
STREAM_WK = 5
STREAM_MASK = 6


def _mix_inplace(z: np.ndarray, t: np.ndarray) -> None:
    np.right_shift(z, np.uint64(30), out=t); np.bitwise_xor(z, t, out=z); np.multiply(z, _M1, out=z)
    np.right_shift(z, np.uint64(27), out=t); np.bitwise_xor(z, t, out=z); np.multiply(z, _M2, out=z)
    np.right_shift(z, np.uint64(31), out=t); np.bitwise_xor(z, t, out=z)


def splitmix64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Draws ``start .. start+count-1`` of one stream as uint64."""
    base = (int(seed) + (stream * _STREAM_STRIDE + start + 1) * int(GOLDEN)) % (1 << 64)
    z = np.arange(count, dtype=np.uint64)
    chunk = 1 << 16
    t = np.empty(min(count, chunk), dtype=np.uint64)
    with np.errstate(over="ignore"):
        for c0 in range(0, count, chunk):
            zz = z[c0:c0 + chunk]
            np.multiply(zz, GOLDEN, out=zz)
            np.add(zz, np.uint64(base), out=zz)
            _mix_inplace(zz, t[:zz.size])
    return z


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, stream: int, count: int, sigma: float, start: int = 0) -> np.ndarray:
    """``count`` N(0, sigma^2) values as bf16 bits, elements ``start..`` of the stream.

    Element ``2k`` takes the cosine branch and ``2k+1`` the sine branch of the
    Box-Muller pair drawn from uniforms ``2k`` and ``2k+1``.
    """
    if count == 0:
        return np.zeros(0, dtype=np.uint16)
    out = np.empty(count, dtype=np.uint16)
    chunk = 1 << 20
    for c0 in range(0, count, chunk):
        c1 = min(count, c0 + chunk)
        out[c0:c1] = _normal_chunk(seed, stream, start + c0, c1 - c0, sigma)
    return out


def _normal_chunk(seed: int, stream: int, start: int, count: int, sigma: float) -> np.ndarray:
    p0 = start // 2
    p1 = (start + count + 1) // 2
    u = splitmix64(seed, stream, 2 * p0, 2 * (p1 - p0))
    u1 = ((u[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    u2 = (u[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * (p1 - p0), dtype=np.float64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    off = start - 2 * p0
    z = z[off:off + count] * sigma
    return f32_to_bf16_bits(z.astype(np.float32))


def rope_table(n_pos: int, rotary_dim: int = 64, theta: float = 1e7):
    """cos/sin tables [n_pos][rotary_dim/2] float32, built in float64, rounded once."""
    half = rotary_dim // 2
    j = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / rotary_dim)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def visibility_mask(S: int, budget: int, seed: int, rows: Optional[np.ndarray] = None,
                    chunk: int = 256) -> np.ndarray:
    """uint8 [len(rows)][S] mask (non-zero = visible); rows default to 0..S-1."""
    if rows is None:
        rows = np.arange(S, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, S), dtype=np.uint8)
    if S == 0:
        return out
    col = np.arange(S, dtype=np.uint64)
    assert S <= (1 << 13), "sort-key tie breaker holds 13 bits of key index"
    for c0 in range(0, rows.size, chunk):
        rr = rows[c0:c0 + chunk]
        for n, i in enumerate(rr):
            if i < budget:
                out[c0 + n, :i + 1] = 1
        big = rr[rr >= budget]
        if big.size == 0:
            continue
        keys = np.empty((big.size, S), dtype=np.uint64)
        for n, i in enumerate(big):
            keys[n] = (splitmix64(seed, STREAM_MASK, int(i) * S, S) & ~np.uint64(0x1FFF)) | col
        keys[col[None, :] >= big[:, None].astype(np.uint64)] = np.uint64(0xFFFFFFFFFFFFFFFF)
        pick = np.argpartition(keys, budget - 2, axis=1)[:, :budget - 1]
        pos = np.nonzero(rr >= budget)[0]
        for n in range(big.size):
            out[c0 + pos[n], pick[n]] = 1
            out[c0 + pos[n], big[n]] = 1
    return out


@dataclasses.dataclass
class Problem:
    """One prefill problem: raw inputs only (bf16 as uint16 bits)."""
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rotary_dim: int
    T: int                 # keys
    q_base: int            # first query position; query rows = T - q_base
    qg: np.ndarray         # [rows][Hq][2][D]  q then gate, per head
    k: np.ndarray          # [T][Hkv][D]
    v: np.ndarray          # [T][Hkv][D]
    q_norm_w: np.ndarray   # [D]
    k_norm_w: np.ndarray   # [D]
    cos: np.ndarray        # [n_pos][R/2] float32
    sin: np.ndarray        # [n_pos][R/2] float32
    mask: Optional[np.ndarray] = None   # [rows][T] uint8 or None
    rms_eps: float = 1e-6
    seed: int = 0
    causal: bool = True    # False: bidirectional pass (every row sees keys 0..T-1)

    @property
    def rows(self) -> int:
        return self.T - self.q_base

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def visible_pairs_per_head(self) -> int:
        if self.mask is not None:
            return int(self.mask.astype(bool).sum())
        if not self.causal:
            return self.rows * self.T
        n = self.rows
        return n * self.q_base + n * (n + 1) // 2

    def flops(self) -> float:
        """Algorithmic FLOPs: 4*D per visible (row, key, q head) triple."""
        return 4.0 * self.head_dim * self.n_q_heads * self.visible_pairs_per_head()

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.qg, self.k, self.v, self.q_norm_w, self.k_norm_w, self.cos, self.sin):
            h.update(np.ascontiguousarray(a).tobytes())
        if self.mask is not None:
            h.update(np.ascontiguousarray(self.mask).tobytes())
        return h.hexdigest()


def make_problem(*, T: int, n_q_heads: int = 24, n_kv_heads: int = 2, head_dim: int = 256,
                 rotary_dim: int = 64, q_base: int = 0, seed: int = 0, q_sigma: float = 1.0,
                 gate_sigma: float = 1.0, kv_sigma: float = 1.0, w_sigma: float = 0.1,
                 mask_budget: Optional[int] = None, theta: float = 1e7, n_pos: Optional[int] = None,
                 causal: bool = True, name: str = "custom") -> Problem:
    """Draws one problem in the fixed order qg(q), qg(gate), K, V, w_q, w_k, mask."""
    rows = T - q_base
    Hq, Hkv, D = n_q_heads, n_kv_heads, head_dim
    # qg rows are the query rows q_base..T-1; each row's values come from the
    # stream positions of its absolute row so a window equals the full pass's rows.
    nq = Hq * D
    q = normal_bf16(seed, STREAM_QG_Q, rows * nq, q_sigma, start=q_base * nq)
    g = normal_bf16(seed, STREAM_QG_GATE, rows * nq, gate_sigma, start=q_base * nq)
    qg = np.empty((rows, Hq, 2, D), dtype=np.uint16)
    qg[:, :, 0, :] = q.reshape(rows, Hq, D)
    qg[:, :, 1, :] = g.reshape(rows, Hq, D)
    k = normal_bf16(seed, STREAM_K, T * Hkv * D, kv_sigma).reshape(T, Hkv, D)
    v = normal_bf16(seed, STREAM_V, T * Hkv * D, kv_sigma).reshape(T, Hkv, D)
    wq = normal_bf16(seed, STREAM_WQ, D, w_sigma)
    wk = normal_bf16(seed, STREAM_WK, D, w_sigma)
    cos, sin = rope_table(max(T, 1) if n_pos is None else n_pos, rotary_dim, theta)
    mask = None
    if mask_budget is not None:
        assert q_base == 0, "masked problems start at q_base 0"
        mask = visibility_mask(T, mask_budget, seed)
    if not causal:
        assert q_base == 0 and mask_budget is None, "a bidirectional pass starts at q_base 0, unmasked"
    return Problem(name=name, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, rotary_dim=rotary_dim,
                   T=T, q_base=q_base, qg=qg, k=k, v=v, q_norm_w=wq, k_norm_w=wk, cos=cos,
                   sin=sin, mask=mask, seed=seed, causal=causal)


@dataclasses.dataclass
class Batch:
    """A packed batch of independent causal sequences of one layer: every
    sequence shares the norm weights and the rotary table (positions 0..len-1
    each); the packed tensors are the sequences' rows back to back."""
    name: str
    seqs: list             # Problem per sequence (shared q_norm_w, k_norm_w, cos, sin)

    @property
    def lens(self):
        return [p.T for p in self.seqs]

    @property
    def total(self) -> int:
        return int(sum(self.lens))

    def _cat(self, attr):
        return np.concatenate([getattr(p, attr) for p in self.seqs], axis=0)

    @property
    def qg(self):
        return self._cat("qg")

    @property
    def k(self):
        return self._cat("k")

    @property
    def v(self):
        return self._cat("v")

    def flops(self) -> float:
        return float(sum(p.flops() for p in self.seqs))


def make_batch(lens, *, n_q_heads: int = 24, n_kv_heads: int = 2, seed: int = 0, gate_sigma: float = 1.0,
               name: str = "batch") -> Batch:
    """Sequence i draws its rows under seed ``seed * 1009 + 1 + i``; the shared
    weights and table come from ``seed`` (a table of max(lens) positions)."""
    n_pos = max([int(x) for x in lens] + [1])
    shared = make_problem(T=1, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, seed=seed, n_pos=n_pos)
    seqs = []
    for i, L in enumerate(lens):
        p = make_problem(T=int(L), n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, seed=seed * 1009 + 1 + i,
                         gate_sigma=gate_sigma, n_pos=n_pos, name=f"{name}[{i}]")
        seqs.append(dataclasses.replace(p, q_norm_w=shared.q_norm_w, k_norm_w=shared.k_norm_w, cos=shared.cos,
                                        sin=shared.sin))
    return Batch(name=name, seqs=seqs)


@dataclasses.dataclass
class SharedPrefix:
    """Branches of one shared prefix: ``prefix`` is the prefix's own causal
    problem (positions 0..P-1); branch i is a window problem (T = P + len_i,
    q_base = P) whose keys 0..P-1 are the prefix's and whose query rows and
    keys P.. are its own.  All share the norm weights and the rotary table."""
    name: str
    prefix: Problem
    branches: list

    @property
    def P(self) -> int:
        return self.prefix.T

    @property
    def lens(self):
        return [b.rows for b in self.branches]

    @property
    def total(self) -> int:
        return int(sum(self.lens))

    @property
    def qg(self):
        return np.concatenate([b.qg for b in self.branches], axis=0)

    @property
    def k(self):
        return np.concatenate([b.k[self.P:] for b in self.branches], axis=0)

    @property
    def v(self):
        return np.concatenate([b.v[self.P:] for b in self.branches], axis=0)

    def flops(self) -> float:
        return float(sum(b.flops() for b in self.branches))


def make_shared_prefix(P: int, lens, *, n_q_heads: int = 24, n_kv_heads: int = 2, seed: int = 0,
                       gate_sigma: float = 1.0, name: str = "shared") -> SharedPrefix:
    """The prefix draws under ``seed``, branch i's rows and keys under
    ``seed * 1009 + 1 + i`` (a table of P + max(lens) positions)."""
    n_pos = P + max([int(x) for x in lens] + [1])
    pre = make_problem(T=max(P, 1), n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, seed=seed, gate_sigma=gate_sigma,
                       n_pos=n_pos, name=f"{name}.prefix")
    if P == 0:
        pre = dataclasses.replace(pre, T=0, qg=pre.qg[:0], k=pre.k[:0], v=pre.v[:0])
    branches = []
    for i, L in enumerate(lens):
        own = make_problem(T=P + int(L), q_base=P, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                           seed=seed * 1009 + 1 + i, gate_sigma=gate_sigma, n_pos=n_pos, name=f"{name}[{i}]")
        branches.append(dataclasses.replace(
            own, k=np.concatenate([pre.k, own.k[P:]], axis=0), v=np.concatenate([pre.v, own.v[P:]], axis=0),
            q_norm_w=pre.q_norm_w, k_norm_w=pre.k_norm_w, cos=pre.cos, sin=pre.sin))
    return SharedPrefix(name=name, prefix=pre, branches=branches)


def batch_lens(n: int, lo: int, hi: int, seed: int):
    """n lengths uniform in [lo, hi] from the counter-based stream (stream 7)."""
    u = splitmix64(seed, 7, 0, n)
    return [int(lo + (int(x) % (hi - lo + 1))) for x in u]


# Packed-batch workload: 16 sequences of 128..2048 tokens (lengths drawn as in
# batch_lens), the 24/2 head geometry; stands in for a serving pack of prompts.
BATCH_CONFIGS = {
    "c6_varlen_16x128_2048": dict(n=16, lo=128, hi=2048, n_q_heads=24, n_kv_heads=2, seed=6),
}


def config_batch(name: str) -> Batch:
    kw = dict(BATCH_CONFIGS[name])
    lens = batch_lens(kw.pop("n"), kw.pop("lo"), kw.pop("hi"), kw["seed"])
    return make_batch(lens, name=name, **kw)


# Shared-prefix workload: one 4096-token prefix continued by 16 branches of
# 128..512 tokens (lengths as in batch_lens), the 24/2 head geometry; stands in
# for a serving request whose candidates share a long prompt.
SHARED_CONFIGS = {
    "c8_shared_4096_16x128_512": dict(P=4096, n=16, lo=128, hi=512, n_q_heads=24, n_kv_heads=2, seed=8),
}


def config_shared(name: str) -> SharedPrefix:
    kw = dict(SHARED_CONFIGS[name])
    lens = batch_lens(kw.pop("n"), kw.pop("lo"), kw.pop("hi"), kw["seed"])
    return make_shared_prefix(kw.pop("P"), lens, name=name, **kw)


# The workloads: (keys, q heads, kv heads, q_base, seed, gate sigma, mask budget, causal).
# c5 is the bidirectional pass (vision-path attention, no causal predicate) at c2's shape.
CONFIGS = {
    "c0_tiny_s64": dict(T=64, n_q_heads=24, n_kv_heads=2, q_base=0, seed=0),
    "c1_dense_s2048": dict(T=2048, n_q_heads=24, n_kv_heads=2, q_base=0, seed=1),
    "c2_dense_s8192_g4": dict(T=8192, n_q_heads=16, n_kv_heads=4, q_base=0, seed=2, gate_sigma=2.0),
    "c3_prefix_t8192_qb1024": dict(T=8192, n_q_heads=24, n_kv_heads=2, q_base=1024, seed=3),
    "c4_masked_s8192": dict(T=8192, n_q_heads=24, n_kv_heads=2, q_base=0, seed=4, mask_budget=2048),
    "c5_bidir_s8192_g4": dict(T=8192, n_q_heads=16, n_kv_heads=4, q_base=0, seed=5, gate_sigma=2.0,
                              causal=False),
    "c7_bidir_s2048": dict(T=2048, n_q_heads=24, n_kv_heads=2, q_base=0, seed=7, causal=False),
}


def config_problem(name: str, **overrides) -> Problem:
    kw = dict(CONFIGS[name])
    kw.update(overrides)
    return make_problem(name=name, **kw)
