"""Pins of the CPU oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with what the mathematics, a library routine, or an
invariant of the method fixes.  ``test_oracle_pins.py`` runs them on the
oracle; ``test_oracle_mutants.py`` runs them on builds of the oracle with one
planted mistake each and requires every mutant to fail at least one pin.

Passages the pins rest on (the QSA kernel page, "feat(qwen4): add the QSA
sparse-attention kernel and its golden", sections "Semantics" and
"Validation", plus its final commit message; the attention-tile page,
"cuda: widen the attention query tile on sm_89 and sm_120", review section
"Kernel change"):
* (1+w) RMSNorm, partial RoPE from a shared table, GQA by repeat-kv,
  q.k/sqrt(256), mask polarity non-zero = visible, fp32 softmax over rounded
  bf16 scores, bf16 weights before the context, sigmoid gate rounded before
  the final product;
* controls: a wrong KV-head mapping and a saturated gate change the output;
* windows: a prefix window equals the matching rows of the full pass.
"""

from __future__ import annotations

import os
import sys

import numpy as np

import synth
from f64_ref import (U, bf, rmsnorm_f64, rope_f64, sdpa_f64, score_max_f64, sigmoid_f64,
                     torch_bf16)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
if GOLDEN not in sys.path:
    sys.path.insert(0, GOLDEN)


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _problem(T, Hq=4, Hkv=2, q_base=0, seed=0, mask_budget=None, gate_sigma=1.0, causal=True):
    return synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, q_base=q_base, seed=seed,
                              mask_budget=mask_budget, gate_sigma=gate_sigma, causal=causal)


# --------------------------------------------------------------------------
# bf16 round to nearest even
# --------------------------------------------------------------------------

def pin_bf16_golden_cases(o):
    """Hand-derived IEEE 754 roundTiesToEven cases (tests/golden/bf16_rne_cases.txt)."""
    pats, want = [], []
    with open(os.path.join(GOLDEN, "bf16_rne_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            a, b = line.split()
            pats.append(int(a, 16))
            want.append(int(b, 16))
    x = np.array(pats, dtype=np.uint32).view(np.float32)
    got = o.bf16_round(x).astype(np.uint32)
    want = np.array(want, dtype=np.uint32)
    isnan = (want & 0x7F80) == 0x7F80
    isnan &= (want & 0x007F) != 0
    ok = np.where(isnan, ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0), got == want)
    assert ok.all(), f"bf16 RNE golden mismatch at {np.nonzero(~ok)[0].tolist()}"


def pin_bf16_vs_torch(o, n=1 << 20):
    """Round-to-nearest-even against torch's float32 -> bfloat16 cast (a library routine)."""
    import torch
    r = _rng(1)
    u = r.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    # Every exponent, and the bits right around the rounding boundary.
    e = np.arange(256, dtype=np.uint32) << np.uint32(23)
    edge = np.array([0x7FFF, 0x8000, 0x8001, 0x17FFF, 0x18000, 0x18001, 0x0, 0xFFFF], np.uint32)
    extra = (e[:, None] | edge[None, :]).ravel()
    u = np.concatenate([u, extra, extra | np.uint32(0x80000000)])
    x = u.view(np.float32)
    got = o.bf16_round(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan]), "bf16 rounding differs from torch"
    assert (((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0)).all(), "NaN not kept"


# --------------------------------------------------------------------------
# (1+w) RMSNorm and partial RoPE
# --------------------------------------------------------------------------

def _norm_only(o, x, w, eps=1e-6):
    one = np.ones(32, np.float32)
    zero = np.zeros(32, np.float32)
    return o.norm_rope(x, w, one, zero, rotary_dim=0, eps=eps)


def pin_norm_closed_form(o):
    """Constant row c*1 gives c/sqrt(c^2+eps)*(1+w) per element (to one bf16 rounding)."""
    D = 256
    for c, wv in [(1.0, 0.0), (3.5, 0.0), (-2.0, 0.0), (1e-3, 0.0), (2.0, 0.5), (0.75, -1.0),
                  (1e-3, 0.25)]:
        x = _bf16_bits(np.full(D, c))
        w = _bf16_bits(np.full(D, wv))
        cq, wq = bf(x)[0], bf(w)[0]
        want = cq / np.sqrt(cq * cq + 1e-6) * (1.0 + wq)
        got = bf(_norm_only(o, x, w))
        tol = 2 * U * abs(want) + 1e-30
        assert np.all(np.abs(got - want) <= tol), f"norm of constant {c} (w={wv}): {got[0]} vs {want}"


def pin_norm_f64(o):
    """Random rows against the float64 (1+w) RMSNorm, within two bf16 roundings."""
    r = _rng(2)
    for trial in range(20):
        x = _bf16_bits(r.normal(0, [0.01, 1.0, 30.0][trial % 3], 256))
        w = _bf16_bits(r.normal(0, 0.1, 256))
        want = rmsnorm_f64(bf(x), bf(w), 1e-6)
        got = bf(_norm_only(o, x, w))
        assert np.all(np.abs(got - want) <= 2 * U * np.abs(want) + 1e-30), "norm vs float64"


def pin_rope_identity_at_zero(o):
    """Position 0 has cos 1, sin 0: the rotation is the identity, exactly."""
    r = _rng(3)
    cos, sin = synth.rope_table(4)
    for _ in range(10):
        x = _bf16_bits(r.normal(0, 1, 256))
        w = _bf16_bits(r.normal(0, 0.1, 256))
        got = o.norm_rope(x, w, cos[0], sin[0])
        assert np.array_equal(got, _norm_only(o, x, w)), "RoPE at position 0 is not the identity"


def pin_rope_f64_rotation(o):
    """The first 64 dims are the exact complex rotation of pairs (j, j+32); the rest pass through."""
    r = _rng(4)
    n_pos = 9000
    cos, sin = synth.rope_table(n_pos)
    for pos in [1, 2, 7, 100, 1023, 2054, 4097, 8191, 8999]:
        x = _bf16_bits(r.normal(0, 1, 256))
        w = _bf16_bits(r.normal(0, 0.1, 256))
        nrm = bf(_norm_only(o, x, w))
        got = bf(o.norm_rope(x, w, cos[pos], sin[pos]))
        want = rope_f64(nrm, pos)
        assert np.array_equal(got[64:], nrm[64:]), "dims past the rotary slice changed"
        a, b = np.abs(nrm[:32]), np.abs(nrm[32:64])
        # cos/sin, two products and the sum are each rounded to bf16.
        tol = 4 * U * np.concatenate([a + b, a + b]) + 1e-6
        assert np.all(np.abs(got[:64] - want[:64]) <= tol), f"RoPE vs float64 rotation at {pos}"


def pin_rope_relative_position(o):
    """Rotated q.k depends only on the position difference (a property of a rotation)."""
    r = _rng(5)
    cos, sin = synth.rope_table(9000)
    for trial in range(6):
        q = _bf16_bits(r.normal(0, 1, 256))
        k = _bf16_bits(r.normal(0, 1, 256))
        w = _bf16_bits(r.normal(0, 0.1, 256))
        a, b = [(10, 3), (500, 20), (3000, 2999), (7000, 100), (64, 0), (8000, 4000)][trial]
        vals = []
        for shift in [0, 17, 777]:
            qr = bf(o.norm_rope(q, w, cos[a + shift], sin[a + shift]))
            kr = bf(o.norm_rope(k, w, cos[b + shift], sin[b + shift]))
            vals.append(float(np.dot(qr[:64], kr[:64])))
        nq = bf(_norm_only(o, q, w))[:64]
        nk = bf(_norm_only(o, k, w))[:64]
        tol = 12 * U * float(np.dot(np.abs(nq), np.abs(nk))) + 1e-3
        assert max(vals) - min(vals) <= tol, f"rotary score not shift-invariant: {vals}"
        # And it is the rotation of the pair, not a reflection: the f64 value agrees.
        want = float(np.dot(rope_f64(nq, a), rope_f64(nk, b)))
        assert abs(vals[0] - want) <= tol, f"rotary score {vals[0]} vs float64 {want}"


def _prologue_err(n, rotary_dim=64):
    """Per-element bound on |prepared - exact| for a vector whose exact (float64)
    normed value is n: the norm's one rounding (plus fp32 noise) on every dim,
    and on the rotary pairs the roundings of cos/sin, of both products and of
    the sum (relative to |a| + |b| of the pair)."""
    half = rotary_dim // 2
    e = 2 * U * np.abs(n)
    ab = np.abs(n[..., :half]) + np.abs(n[..., half:rotary_dim])
    e[..., :half] = 5 * U * ab
    e[..., half:rotary_dim] = 5 * U * ab
    return e + 1e-30


def pin_prepare_keys_f64(o):
    """Each prepared key is the float64 (1+w) RMSNorm of its own raw row, rotated at
    the key's own position, for its own KV head: positions and heads come from the
    raw inputs here, not from the oracle (the QSA kernel page, "Semantics": every
    key is normed and partially rotated once per KV head at its position)."""
    for T, Hkv, seed in [(300, 3, 19), (70, 2, 20)]:
        p = _problem(T, 2 * Hkv, Hkv, seed=seed)
        got = bf(o.prepare_keys(p))                          # [Hkv][T][D]
        n = rmsnorm_f64(bf(p.k), bf(p.k_norm_w), 1e-6)       # [T][Hkv][D]
        want = rope_f64(n, np.arange(T)[:, None]).transpose(1, 0, 2)
        tol = _prologue_err(n).transpose(1, 0, 2)
        bad = np.abs(got - want) > tol
        assert not bad.any(), (f"prepared keys vs float64 norm + rotation at the key's position and head: "
                               f"{bad.sum()} of {bad.size} (T={T}, Hkv={Hkv})")


def pin_prepare_queries_f64(o):
    """Each prepared query is the float64 (1+w) RMSNorm of the q half of its own head's
    slice of the fused row, rotated at absolute position q_base + i."""
    for T, Hq, Hkv, qb, seed in [(90, 6, 2, 0, 21), (300, 4, 2, 128, 22)]:
        p = _problem(T, Hq, Hkv, q_base=qb, seed=seed)
        got = bf(o.prepare_queries(p))                       # [rows][Hq][D]
        n = rmsnorm_f64(bf(p.qg[:, :, 0, :]), bf(p.q_norm_w), 1e-6)
        want = rope_f64(n, (qb + np.arange(p.rows))[:, None])
        bad = np.abs(got - want) > _prologue_err(n)
        assert not bad.any(), f"prepared queries vs float64 (q_base={qb}): {bad.sum()} of {bad.size}"


def pin_attention_from_raw_vs_sdpa(o):
    """Whole path from the raw inputs: float64 norm + rotation of raw q and k at
    absolute positions, then float64 scaled-dot-product attention (torch, its own
    GQA mapping and mask), against the oracle's ungated context.  Bound: the three
    roundings after the scores (as in pin_attention_vs_sdpa) plus the prologue's:
    a score moves by at most ds = sum_d (eq|k| + |q|ek + eq ek) / 16, which moves a
    weight by a factor within exp(+-2 max ds)."""
    for n_, (T, Hq, Hkv, qb, mb) in enumerate(_GEOMS):
        p = _problem(T, Hq, Hkv, q_base=qb, seed=200 + n_, mask_budget=mb)
        r = o.attention(p, want_ctx=True)
        nq = rmsnorm_f64(bf(p.qg[:, :, 0, :]), bf(p.q_norm_w), 1e-6)          # [rows][Hq][D]
        nk = rmsnorm_f64(bf(p.k), bf(p.k_norm_w), 1e-6)                       # [T][Hkv][D]
        q64 = rope_f64(nq, (qb + np.arange(p.rows))[:, None])
        k64 = rope_f64(nk, np.arange(T)[:, None]).transpose(1, 0, 2)          # [Hkv][T][D]
        eq, ek = _prologue_err(nq), _prologue_err(nk).transpose(1, 0, 2)
        v = bf(p.v)
        want = sdpa_f64(q64, k64, v, qb, p.mask)
        absv = sdpa_f64(q64, k64, np.abs(v), qb, p.mask)
        smax = score_max_f64(q64, k64, qb, p.mask)
        G = Hq // Hkv
        kk, ekk = np.repeat(k64, G, axis=0), np.repeat(ek, G, axis=0)         # [Hq][T][D]
        ds = (np.einsum("rhd,htd->rht", eq, np.abs(kk)) + np.einsum("rhd,htd->rht", np.abs(q64), ekk)
              + np.einsum("rhd,htd->rht", eq, ekk)) / 16.0
        dmax = ds.max(axis=-1)                                                # over keys (a bound)
        got = bf(r["ctx"]).reshape(want.shape)
        tol = (1.5 * (U * np.abs(want) + U * (1.0 + 2.0 * smax[..., None]) * absv)
               + 1.1 * np.expm1(2.0 * dmax)[..., None] * absv + 1e-7)
        bad = np.abs(got - want) > tol
        assert not bad.any(), (f"context from raw inputs vs float64 attention, geometry {n_}: "
                               f"{bad.sum()} of {bad.size}")


# --------------------------------------------------------------------------
# Attention core and gate
# --------------------------------------------------------------------------

_GEOMS = [
    # (T, Hq, Hkv, q_base, mask_budget)
    (1, 2, 1, 0, None),
    (5, 4, 2, 0, None),
    (37, 6, 2, 0, None),
    (64, 24, 2, 0, None),
    (48, 4, 4, 16, None),
    (70, 8, 2, 0, 9),
]


def pin_attention_vs_sdpa(o):
    """Ungated context against float64 scaled-dot-product attention on the oracle's
    own prepared q/k (library routine with its own GQA mapping and mask handling);
    the prepared q/k themselves are pinned from the raw inputs above.

    First-order bound from the three remaining bf16 roundings: score (perturbs the
    weights by at most 2*U*max|s|), weight (U), context (U)."""
    for n, (T, Hq, Hkv, qb, mb) in enumerate(_GEOMS):
        p = _problem(T, Hq, Hkv, q_base=qb, seed=100 + n, mask_budget=mb)
        r = o.attention(p, want_ctx=True)
        qp = bf(o.prepare_queries(p))
        kp = bf(o.prepare_keys(p))
        v = bf(p.v)
        want = sdpa_f64(qp, kp, v, qb, p.mask)
        absv = sdpa_f64(qp, kp, np.abs(v), qb, p.mask)
        smax = score_max_f64(qp, kp, qb, p.mask)
        got = bf(r["ctx"]).reshape(want.shape)
        tol = 1.5 * (U * np.abs(want) + U * (1.0 + 2.0 * smax[..., None]) * absv) + 1e-7
        bad = np.abs(got - want) > tol
        assert not bad.any(), (f"context vs float64 attention, geometry {n}: "
                               f"{bad.sum()} of {bad.size}, worst {np.max(np.abs(got - want) - tol)}")


def pin_bidirectional_vs_sdpa(o):
    """Bidirectional pass (no causal predicate; the vision-path variant of the attention-tile page):
    ungated context against float64 attention over every key, same bound as above."""
    for n, (T, Hq, Hkv) in enumerate([(1, 2, 1), (5, 4, 2), (37, 6, 2), (70, 8, 2)]):
        p = _problem(T, Hq, Hkv, seed=140 + n, causal=False)
        r = o.attention(p, want_ctx=True)
        qp = bf(o.prepare_queries(p))
        kp = bf(o.prepare_keys(p))
        v = bf(p.v)
        want = sdpa_f64(qp, kp, v, 0, causal=False)
        absv = sdpa_f64(qp, kp, np.abs(v), 0, causal=False)
        smax = score_max_f64(qp, kp, 0, causal=False)
        got = bf(r["ctx"]).reshape(want.shape)
        tol = 1.5 * (U * np.abs(want) + U * (1.0 + 2.0 * smax[..., None]) * absv) + 1e-7
        bad = np.abs(got - want) > tol
        assert not bad.any(), (f"bidirectional context vs float64 attention, geometry {n}: "
                               f"{bad.sum()} of {bad.size}")


def pin_bidirectional_last_row_equals_causal(o):
    """The last row sees every key in both passes: identical outputs, bit for bit.
    Earlier rows see later keys only in the bidirectional pass, so they differ."""
    for T in [9, 64]:
        pc = _problem(T, 4, 2, seed=150)
        pb = _problem(T, 4, 2, seed=150, causal=False)
        assert np.array_equal(pc.qg, pb.qg) and np.array_equal(pc.k, pb.k)
        oc, ob = o.attention(pc), o.attention(pb)
        assert np.array_equal(oc[-1], ob[-1]), f"last row, T={T}"
        assert not np.array_equal(oc[0], ob[0]), f"row 0 should see later keys, T={T}"


def pin_row0_closed_form(o):
    """Row 0 sees key 0 alone: its weight is exactly 1, so out = bf16(v0 * bf16(sigmoid(g)))."""
    for seed, gs in [(7, 1.0), (8, 2.0), (9, 4.0)]:
        p = _problem(8, 6, 2, seed=seed, gate_sigma=gs)
        out = bf(o.attention(p, rows=[0]))[0].reshape(6, 256)
        g = bf(p.qg[0, :, 1, :])
        sg = torch_bf16(sigmoid_f64(g))
        v0 = np.repeat(bf(p.v[0]), 3, axis=0)
        want = torch_bf16(v0 * sg)
        diff = out != want
        # sigmoid is evaluated in fp32 by the oracle: a bf16 tie within a few fp32
        # ulps may flip; allow a handful of one-ulp flips, nothing else.
        assert diff.sum() <= 2, f"row 0 closed form: {diff.sum()} mismatches"
        if diff.any():
            assert np.all(np.abs(out[diff] - want[diff]) <= 2 * U * np.abs(want[diff]))


def pin_gate_closed_forms(o):
    """Gate logit 0 halves the context exactly; a saturated logit (32) leaves it unchanged."""
    p = _problem(40, 4, 2, seed=11)
    base = o.attention(p, want_ctx=True)
    for gval, factor in [(0.0, 0.5), (32.0, 1.0)]:
        q = p.qg.copy()
        q[:, :, 1, :] = _bf16_bits(gval)
        pp = synth.Problem(**{**p.__dict__, "qg": q})
        got = bf(o.attention(pp))
        assert np.array_equal(got, bf(base["ctx"]) * factor), f"gate {gval}"


def pin_one_hot_v_zero_pattern(o):
    """With one-hot values the context is each key's weight: hidden keys give exactly
    +0 and visible keys a positive weight (causal, and causal AND mask)."""
    for mb in [None, 5]:
        T, Hq, Hkv = 40, 4, 2
        p = _problem(T, Hq, Hkv, seed=12, mask_budget=mb)
        v = np.zeros((T, Hkv, 256), np.float32)
        for j in range(T):
            v[j, :, j] = 1.0
        q = p.qg.copy()
        q[:, :, 1, :] = _bf16_bits(32.0)
        pp = synth.Problem(**{**p.__dict__, "qg": q, "v": _bf16_bits(v)})
        got = bf(o.attention(pp)).reshape(T, Hq, 256)[:, :, :T]
        vis = np.tril(np.ones((T, T), bool))
        if p.mask is not None:
            vis &= p.mask != 0
        assert np.all(got[~np.broadcast_to(vis[:, None, :], got.shape)] == 0.0), "hidden key leaked"
        assert np.all(got[np.broadcast_to(vis[:, None, :], got.shape)] > 0.0), "visible key dropped"
        assert not np.signbit(got).any(), "negative zero"


def pin_gqa_copy(o):
    """Hkv=2 with G=3 equals Hkv=6 with G=1 when each KV head is copied 3 times."""
    p = _problem(33, 6, 2, seed=13)
    out = o.attention(p)
    k6 = np.repeat(p.k, 3, axis=1)
    v6 = np.repeat(p.v, 3, axis=1)
    p6 = synth.Problem(**{**p.__dict__, "n_kv_heads": 6, "k": k6, "v": v6})
    assert np.array_equal(out, o.attention(p6)), "GQA mapping is not repeat-kv"


def pin_prefix_equals_full(o):
    """A window starting at q_base reproduces the full pass's rows bit for bit."""
    full = _problem(50, 4, 2, seed=14)
    out = o.attention(full)
    for qb in [16, 32, 49]:
        w = synth.make_problem(T=50, n_q_heads=4, n_kv_heads=2, q_base=qb, seed=14)
        assert np.array_equal(w.qg, full.qg[qb:])
        assert np.array_equal(o.attention(w), out[qb:]), f"window at {qb}"


def pin_mask_all_visible_equals_dense(o):
    """An all-visible mask is plain causal attention, bit for bit."""
    p = _problem(45, 4, 2, seed=15)
    pm = synth.Problem(**{**p.__dict__, "mask": np.ones((45, 45), np.uint8) * 7})
    assert np.array_equal(o.attention(p), o.attention(pm))


def pin_hidden_row_is_zero(o):
    """A row with no visible key outputs zeros."""
    p = _problem(20, 4, 2, seed=16, mask_budget=4)
    m = p.mask.copy()
    m[7, :] = 0
    m[12, :13] = 0
    pm = synth.Problem(**{**p.__dict__, "mask": m})
    out = bf(o.attention(pm))
    assert np.all(out[7] == 0) and np.all(out[12] == 0)
    assert np.all(np.abs(out[8]).sum() > 0)


def pin_weight_row_sums(o):
    """The bf16 weights of each row-head sum to 1 within U (each weight rounds by <= U*w)."""
    p = _problem(300, 4, 2, seed=17)
    r = o.attention(p, rows=[0, 1, 2, 63, 64, 150, 299], want_wsum=True)
    assert np.all(np.abs(r["wsum"] - 1.0) <= U + 1e-6), r["wsum"]
    p = _problem(300, 4, 2, seed=18, mask_budget=32)
    r = o.attention(p, rows=[31, 32, 200, 299], want_wsum=True)
    assert np.all(np.abs(r["wsum"] - 1.0) <= U + 1e-6), r["wsum"]


def pin_frozen_regression(o):
    """Frozen oracle output for a tiny problem (tests/golden/oracle_s8_regression.txt),
    written by tests/golden/make_golden.py; a change here must be deliberate."""
    import make_golden
    p = make_golden.problem()
    want = make_golden.read()
    assert np.array_equal(o.attention(p), want), "oracle drifted from its frozen output"


# --------------------------------------------------------------------------
# The other reading of the score's dot product (summed in double)
# --------------------------------------------------------------------------

def _scores_two_ways(qp, kp, G):
    """bf16 scores (float64 values) of every (row, head, key) from prepared
    queries [rows][Hq][D] and keys [Hkv][T][D] (float64 values of bf16): summed
    in ascending order in float32, and exactly in float64 then rounded once to
    float32; each then rounded to bf16 by torch's round-to-nearest-even cast."""
    rows, Hq, D = qp.shape
    kk = np.repeat(kp, G, axis=0).astype(np.float32)               # [Hq][T][D]
    q32 = qp.astype(np.float32)
    serial = np.zeros((rows, Hq, kk.shape[1]), np.float32)
    for d in range(D):
        serial = (serial + q32[:, :, d][:, :, None] * kk[None, :, :, d]).astype(np.float32)
    exact = np.einsum("rhd,htd->rht", qp, kk.astype(np.float64)).astype(np.float32)
    return torch_bf16(serial.astype(np.float64)), torch_bf16(exact.astype(np.float64))


def pin_score_f64_vs_sdpa(o):
    """The double-summed reading passes the float64 attention pin's bound too."""
    for n, (T, Hq, Hkv, qb, mb) in enumerate(_GEOMS):
        p = _problem(T, Hq, Hkv, q_base=qb, seed=100 + n, mask_budget=mb)
        r = o.attention(p, want_ctx=True, score_f64=True)
        qp, kp, v = bf(o.prepare_queries(p)), bf(o.prepare_keys(p)), bf(p.v)
        want = sdpa_f64(qp, kp, v, qb, p.mask)
        absv = sdpa_f64(qp, kp, np.abs(v), qb, p.mask)
        smax = score_max_f64(qp, kp, qb, p.mask)
        got = bf(r["ctx"]).reshape(want.shape)
        tol = 1.5 * (U * np.abs(want) + U * (1.0 + 2.0 * smax[..., None]) * absv) + 1e-7
        assert not (np.abs(got - want) > tol).any(), f"score_f64 context vs float64 attention, geometry {n}"


def pin_score_readings_agree_unless_a_score_rounds_apart(o):
    """The two readings give bit-identical row-heads wherever every visible key's
    bf16 score is the same both ways (scores recomputed here in numpy), and
    differ only in row-heads holding a key whose two scores differ."""
    for n, (T, Hq, Hkv, qb, mb) in enumerate(_GEOMS + [(300, 8, 2, 0, None), (200, 16, 1, 64, None)]):
        p = _problem(T, Hq, Hkv, q_base=qb, seed=300 + n, mask_budget=mb)
        a = o.attention(p).reshape(p.rows, Hq, -1)
        b = o.attention(p, score_f64=True).reshape(p.rows, Hq, -1)
        qp, kp = bf(o.prepare_queries(p)), bf(o.prepare_keys(p))
        s0, s1 = _scores_two_ways(qp, kp, Hq // Hkv)
        vis = np.arange(T)[None, :] <= (qb + np.arange(p.rows))[:, None]
        if p.mask is not None:
            vis &= np.asarray(p.mask) != 0
        apart = ((s0 != s1) & vis[:, None, :]).any(axis=-1)             # [rows][Hq]
        same = (a == b).all(axis=-1)
        assert same[~apart].all(), f"geometry {n}: the readings differ where every score agrees"


def pin_score_f64_rounds_a_near_tie_up(o):
    """A case found by a parity sweep (a 1280-token prefix, a 267-token branch,
    48/6 heads): row 202, head 3's heaviest key (weight 0.028) has the exact
    dot product 69.750007, just above the bf16 tie between 69.5 and 70.  The
    ascending fp32 sum rounds to 69.5, the double sum to 70: the heaviest key's
    weight rises by about exp(0.5/16) and the row-head moves."""
    sp = synth.make_shared_prefix(1280, [45, 236, 195, 267], n_q_heads=48, n_kv_heads=6, seed=518)
    b = sp.branches[3]
    row = np.array([202], np.int32)
    r0 = o.attention(b, rows=row, want_weights=True)
    r1 = o.attention(b, rows=row, want_weights=True, score_f64=True)
    w0, w1 = r0["weights"][0, 3], r1["weights"][0, 3]
    j = int(np.argmax(w0))
    assert j == 600, j
    ratio = float(w1[j] / w0[j])
    assert 1.025 < ratio < 1.04, ratio                                  # exp(1/32) = 1.0317, renormalised
    assert not np.array_equal(r0["out"].reshape(48, -1)[3], r1["out"].reshape(48, -1)[3])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
