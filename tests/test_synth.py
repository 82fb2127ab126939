"""The seeded input generator: determinism, slicing, distributions, mask recipe (CPU)."""

import numpy as np
import pytest

import synth


def test_splitmix_reference_values():
    # SplitMix64 seeded with 0: the published first outputs of the generator.
    got = synth.splitmix64(0, 0, 0, 3)
    assert [int(x) for x in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_slices():
    a = synth.normal_bf16(5, synth.STREAM_K, 5000, 1.0)
    for s, n in [(0, 1), (1, 7), (1001, 2000), (4999, 1)]:
        assert np.array_equal(synth.normal_bf16(5, synth.STREAM_K, n, 1.0, start=s), a[s:s + n])


def test_window_rows_match_full_pass():
    full = synth.make_problem(T=300, seed=9)
    win = synth.make_problem(T=300, q_base=128, seed=9)
    assert np.array_equal(win.qg, full.qg[128:])
    assert np.array_equal(win.k, full.k) and np.array_equal(win.v, full.v)


def test_distributions():
    x = synth.bf16_bits_to_f32(synth.normal_bf16(1, 0, 1 << 20, 2.0)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 2.0) < 0.01
    assert abs(((x / 2.0) ** 4).mean() - 3.0) < 0.05          # Gaussian kurtosis


def test_rope_table_values():
    cos, sin = synth.rope_table(3000)
    for p, j in [(0, 0), (1, 0), (2054, 3), (2999, 31)]:
        ang = p * 1e7 ** (-2 * j / 64)
        assert cos[p, j] == np.float32(np.cos(ang)) and sin[p, j] == np.float32(np.sin(ang))


def test_mask_recipe():
    S, budget = 600, 64
    m = synth.visibility_mask(S, budget, seed=4)
    assert m.dtype == np.uint8 and m.shape == (S, S)
    assert not np.triu(m, 1).any(), "a future key is visible"
    assert m.diagonal().all()
    assert np.array_equal(m.sum(1), np.minimum(np.arange(S) + 1, budget))
    # Row subsets regenerate the same rows.
    rows = np.array([0, 63, 64, 599])
    assert np.array_equal(synth.visibility_mask(S, budget, seed=4, rows=rows), m[rows])
    # Earlier keys are chosen roughly uniformly.
    frac = m[400:, :300].mean()
    assert abs(frac - (budget - 1) / np.arange(400, 600).mean()) < 0.02


@pytest.mark.parametrize("name", ["c0_tiny_s64"])
def test_config_digest_stable(name):
    p = synth.config_problem(name)
    assert p.qg.shape == (64, 24, 2, 256) and p.k.shape == (64, 2, 256)
    assert p.digest() == synth.config_problem(name).digest()


def test_batch_shares_weights_and_packs_rows():
    b = synth.make_batch([0, 5, 33, 64], n_q_heads=4, n_kv_heads=2, seed=3)
    assert b.lens == [0, 5, 33, 64] and b.total == 102
    assert b.qg.shape == (102, 4, 2, 256) and b.k.shape == (102, 2, 256)
    for p in b.seqs:
        assert np.array_equal(p.q_norm_w, b.seqs[0].q_norm_w) and np.array_equal(p.k_norm_w, b.seqs[0].k_norm_w)
        assert p.cos.shape == (64, 32) and np.array_equal(p.cos, b.seqs[0].cos)
    # sequence i's rows sit at its offset
    assert np.array_equal(b.qg[5:38], b.seqs[2].qg)
    # a sequence's rows do not depend on its neighbours
    b2 = synth.make_batch([7, 5, 33, 64], n_q_heads=4, n_kv_heads=2, seed=3)
    assert np.array_equal(b2.seqs[2].qg, b.seqs[2].qg)


def test_batch_lengths_are_seeded_and_in_range():
    a = synth.batch_lens(64, 128, 2048, 6)
    assert a == synth.batch_lens(64, 128, 2048, 6)
    assert min(a) >= 128 and max(a) <= 2048 and len(set(a)) > 32


def test_shared_prefix_branches_share_the_prefix():
    """Branches of a shared prefix: each is a window over prefix + its own tokens,
    its keys 0..P-1 the prefix's, its query rows and keys after P drawn as a plain
    problem of P + len keys would draw them, and every branch shares the prefix's
    norm weights and table; P = 0 gives the packed batch's sequences."""
    sp = synth.make_shared_prefix(256, [1, 0, 70], n_q_heads=8, n_kv_heads=2, seed=4)
    assert sp.P == 256 and sp.lens == [1, 0, 70] and sp.total == 71
    for i, b in enumerate(sp.branches):
        assert (b.T, b.q_base, b.rows) == (256 + sp.lens[i], 256, sp.lens[i])
        assert np.array_equal(b.k[:256], sp.prefix.k) and np.array_equal(b.v[:256], sp.prefix.v)
        own = synth.make_problem(T=b.T, q_base=256, n_q_heads=8, n_kv_heads=2, seed=4 * 1009 + 1 + i,
                                 n_pos=256 + 70)
        assert np.array_equal(b.qg, own.qg) and np.array_equal(b.k[256:], own.k[256:])
        assert np.array_equal(b.q_norm_w, sp.prefix.q_norm_w) and np.array_equal(b.cos, sp.prefix.cos)
    assert sp.qg.shape == (71, 8, 2, 256) and sp.k.shape == (71, 2, 256)
    assert np.array_equal(sp.k[1:], sp.branches[2].k[256:])
    b0 = synth.make_batch([5, 3], n_q_heads=8, n_kv_heads=2, seed=9)
    s0 = synth.make_shared_prefix(0, [5, 3], n_q_heads=8, n_kv_heads=2, seed=9)
    for a, b in zip(b0.seqs, s0.branches):
        assert np.array_equal(a.qg, b.qg) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
        assert np.array_equal(a.q_norm_w, b.q_norm_w) and np.array_equal(a.cos, b.cos)
