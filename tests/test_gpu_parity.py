"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerance per bf16 output element: |gpu - oracle| <= 1e-2 + 1e-2 * |oracle|
(the contract), and in addition a value-scaled bound that a wrong row cannot
pass at any length: the deviation measured in quanta of each row-head's own
scale (gpu_util.row_scale_quanta; rms <= 3, each element within 16 quanta
or two bf16 steps of itself).
Index and mask handling are checked bit-exactly (zero patterns, perturbation
invariance, identities), at full size too.  The prologue (norm + RoPE)
reproduces the oracle's arithmetic in the same order, so prepared queries and
keys are compared bit for bit.  With ATTN_PARITY_LOG set, every comparison
appends its record (bound fraction, quanta histogram) to that file.
"""

import os
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        if os.environ.get("ATTN_REQUIRE_GPU") == "1":
            pytest.fail("ATTN_REQUIRE_GPU=1 but no GPU is visible")
        pytest.skip("no GPU")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    _need_gpu()
    import gated_gqa_causal_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


from gpu_util import (DevProblem, bits_to_f32, check_parity, check_parity_either_reading, debug_fp8_encode,  # noqa: E402
                      debug_prepare, gpu_out, make_ctx, parity_record, parity_report, run, to_bits)

_CFG = {}


def cfg(name):
    """A workload's inputs, drawn once per test session (the generator is slow at 8192 tokens)."""
    if name not in _CFG:
        _CFG[name] = synth.config_problem(name)
    return _CFG[name]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_rows(orc, p, rows, threads=8):
    return orc.attention(p, rows=rows, threads=threads)


def sample_rows(n_rows, k=48, seed=0):
    """First/last rows, every tile-boundary neighbourhood in a stride, plus random rows."""
    r = np.random.default_rng(seed)
    s = set(range(min(4, n_rows))) | set(range(max(0, n_rows - 4), n_rows))
    for b in range(0, n_rows, max(64, n_rows // 8)):
        s |= {x for x in (b - 1, b, b + 31, b + 32, b + 63) if 0 <= x < n_rows}
    s |= set(r.integers(0, n_rows, size=k).tolist())
    return np.array(sorted(s), dtype=np.int32)


# --------------------------------------------------------------------------
# Prologue: bit-exact prepared queries and keys (through the test build's hook)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,Hq,Hkv,qb", [(64, 24, 2, 0), (200, 16, 4, 0), (300, 4, 2, 128), (33, 2, 1, 0)])
def test_prologue_bit_exact(orc, T, Hq, Hkv, qb):
    say(f"prologue T={T} Hq={Hq} Hkv={Hkv} q_base={qb}")
    p = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, q_base=qb, seed=T)
    qp, kp = debug_prepare(DevProblem(p), q_base=qb)
    assert np.array_equal(to_bits(kp), orc.prepare_keys(p)), "prepared keys differ"
    assert np.array_equal(to_bits(qp), orc.prepare_queries(p)), "prepared queries differ"


# --------------------------------------------------------------------------
# Whole-output parity at sizes the oracle covers fully
# --------------------------------------------------------------------------

FULL_CASES = [
    # name, make_problem kwargs
    ("c0_tiny_s64", dict(T=64, n_q_heads=24, n_kv_heads=2, seed=0)),
    ("s1", dict(T=1, n_q_heads=24, n_kv_heads=2, seed=5)),
    ("s33_g1", dict(T=33, n_q_heads=2, n_kv_heads=2, seed=6)),
    ("s200_ragged", dict(T=200, n_q_heads=24, n_kv_heads=2, seed=7)),
    ("s333_g4", dict(T=333, n_q_heads=16, n_kv_heads=4, seed=8, gate_sigma=2.0)),
    ("s130_g16", dict(T=130, n_q_heads=32, n_kv_heads=2, seed=9)),
    ("s97_g6", dict(T=97, n_q_heads=6, n_kv_heads=1, seed=10)),
    ("prefix_t300_qb128", dict(T=300, n_q_heads=24, n_kv_heads=2, q_base=128, seed=11)),
    ("prefix_t513_qb256", dict(T=513, n_q_heads=8, n_kv_heads=2, q_base=256, seed=12)),
    ("masked_s300_b40", dict(T=300, n_q_heads=24, n_kv_heads=2, seed=13, mask_budget=40)),
    ("masked_s257_b7_g4", dict(T=257, n_q_heads=8, n_kv_heads=2, seed=14, mask_budget=7)),
    ("bidir_s64", dict(T=64, n_q_heads=24, n_kv_heads=2, seed=15, causal=False)),
    ("bidir_s1", dict(T=1, n_q_heads=4, n_kv_heads=2, seed=16, causal=False)),
    ("bidir_s200_ragged", dict(T=200, n_q_heads=16, n_kv_heads=4, seed=17, gate_sigma=2.0, causal=False)),
    ("bidir_s333_g6", dict(T=333, n_q_heads=6, n_kv_heads=1, seed=18, causal=False)),
]


def _random_cases(n=40, seed=2026):
    """Seeded random small problems: length 1..700 (ragged tails), a GQA shape with
    G in 1..16, a q_base multiple of 128 below T for a third of the causal ones, a
    mask of random budget for a third of the q_base = 0 ones, and bidirectional
    passes; every element against the oracle."""
    rng = np.random.default_rng(seed)
    shapes = [(24, 2), (16, 4), (8, 8), (32, 2), (6, 1), (12, 3), (40, 5), (2, 2), (48, 6), (16, 1)]
    cases = []
    for i in range(n):
        T = int(rng.integers(1, 701))
        Hq, Hkv = shapes[int(rng.integers(len(shapes)))]
        kw = dict(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=100 + i, gate_sigma=float(rng.choice([1.0, 2.0])))
        kind = int(rng.integers(4))
        if kind == 1 and T > 128:
            kw["q_base"] = 128 * int(rng.integers(1, (T - 1) // 128 + 1))
        elif kind == 2:
            kw["mask_budget"] = int(rng.integers(1, max(2, T)))
        elif kind == 3:
            kw["causal"] = False
        cases.append((f"r{i:02d}_T{T}_{Hq}x{Hkv}_k{kind}", kw))
    return cases


def _random_larger_cases(n=30, seed=11):
    """Seeded random problems of 1..4096 keys over eleven GQA shapes (up to 64
    query heads), prefix windows, masks of random budget and bidirectional
    passes; sampled rows (tile boundaries, first and last) against the oracle."""
    rng = np.random.default_rng(seed)
    shapes = [(24, 2), (16, 4), (8, 8), (32, 2), (6, 1), (12, 3), (40, 5), (2, 2), (48, 6), (16, 1), (64, 4)]
    cases = []
    for i in range(n):
        T = int(rng.integers(1, 4097))
        Hq, Hkv = shapes[int(rng.integers(len(shapes)))]
        kw = dict(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=7000 + i, gate_sigma=float(rng.choice([1.0, 2.0])))
        kind = int(rng.integers(4))
        if kind == 1 and T > 128:
            kw["q_base"] = 128 * int(rng.integers(1, (T - 1) // 128 + 1))
        elif kind == 2:
            kw["mask_budget"] = int(rng.integers(1, max(2, T)))
        elif kind == 3:
            kw["causal"] = False
        cases.append((f"L{i:02d}_T{T}_{Hq}x{Hkv}_k{kind}", kw))
    return cases


@pytest.mark.parametrize("name,kw", _random_larger_cases(), ids=[c[0] for c in _random_larger_cases()])
def test_parity_random_larger_shapes(orc, name, kw):
    say(f"parity_random_larger {name} {kw}")
    p = synth.make_problem(name=name, **kw)
    got = gpu_out(p)
    rows = sample_rows(p.rows, k=16, seed=len(name))
    rec = check_parity_either_reading(orc, p, got[rows], f"random larger {name}", rows=rows)
    say(f"  {rec}")


@pytest.mark.parametrize("name,kw", _random_cases(), ids=[c[0] for c in _random_cases()])
def test_parity_random_shapes(orc, name, kw):
    say(f"parity_random {name} {kw}")
    p = synth.make_problem(name=name, **kw)
    got = gpu_out(p)
    rec = check_parity_either_reading(orc, p, got, f"random {name}")
    say(f"  {rec}")


@pytest.mark.parametrize("name,kw", FULL_CASES, ids=[c[0] for c in FULL_CASES])
def test_parity_full(orc, name, kw):
    say(f"parity_full {name} {kw}")
    p = synth.make_problem(name=name, **kw)
    got = gpu_out(p)
    want = orc.attention(p, threads=8)
    rec = parity_record(f"full {name}", got, want, p.n_q_heads)
    say(f"  {rec}")
    check_parity(rec)


def test_parity_full_block_sparse_mask(orc):
    """Every row of a masked pass whose mask hides whole (64-row block, 32-key
    tile) pairs: about 30% of each block's causal tiles, plus a quarter of the
    remaining keys.  The walks (up to about 100 tiles) skip tiles and run past
    the 32- and 64-entry boundaries of the tile list; all rows against the
    oracle (a row whose keys are all hidden gives zeros)."""
    T = 4096
    say(f"parity_full block-sparse mask T={T}")
    p = synth.make_problem(name="blocksparse", T=T, n_q_heads=8, n_kv_heads=2, seed=43)
    rng = np.random.default_rng(43)
    mask = (rng.random((T, T)) >= 0.25).astype(np.uint8)
    nrb, ntile = (T + 63) // 64, (T + 31) // 32
    off = rng.random((nrb, ntile)) < 0.3
    off[:, 0] = False                                # row 0 keeps key 0 (no empty row block)
    for rb in range(nrb):
        for t in np.nonzero(off[rb])[0]:
            mask[64 * rb:64 * rb + 64, 32 * t:32 * t + 32] = 0
    pm = synth.Problem(**{**p.__dict__, "mask": mask})
    got = gpu_out(pm)
    want = orc.attention(pm, threads=8)
    rec = parity_record("full block-sparse", got, want, pm.n_q_heads)
    say(f"  {rec}")
    check_parity(rec)


def test_host_schedule_table_equals_the_snake():
    """The same pass under the two work schedules: S=8192, 24/2 (768 work items on 256
    compute units, where the context's launch takes the host-planned table) through
    attn_prefill_gated, and through the allocation-free entry point, which always
    follows the snake order; bit-identical (an item computes the same on any
    workgroup, in any order)."""
    import gated_gqa_causal_amd as ga
    p = synth.Problem(**{**cfg("c4_masked_s8192").__dict__, "mask": None})
    say("schedule table vs snake at S=8192 24/2")
    dp = DevProblem(p)
    ctx = make_ctx(p)
    table = to_bits(run(ctx, dp))
    ctx.close()
    out = torch.empty((p.T, p.n_q_heads * 256), dtype=torch.bfloat16, device="cuda")
    geom = ga.geometry(p.n_q_heads, p.n_kv_heads, p.T, p.rms_eps)
    inp = ga.attn_inputs(dp.qg.data_ptr(), dp.k.data_ptr(), dp.v.data_ptr(), dp.wq.data_ptr(), dp.wk.data_ptr(),
                         dp.cos.data_ptr(), dp.sin.data_ptr(), dp.cos.shape[0])
    assert ga.attn_prefill_gated_noalloc(geom, inp, p.T, out.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream) == ga.ATTN_OK
    torch.cuda.synchronize()
    snake = to_bits(out)
    same = np.array_equal(table, snake)
    say(f"  bit-identical: {same}")
    assert same


def test_host_schedule_without_xcd_grouping(orc):
    """T=4096 with 48/6 heads (six KV heads do not divide the eight XCDs, so the work
    is planned over all workgroups item by item): at q_base 0 (768 items) and 1024 (576)
    the launches take host-planned tables.  Sampled rows match the oracle, the window's
    rows equal the full pass's bit for bit, and the full pass equals the
    allocation-free entry point's (the snake order) bit for bit."""
    import gated_gqa_causal_amd as ga
    say("schedule table without XCD grouping, T=4096 48/6")
    p = synth.make_problem(name="sched_48_6", T=4096, n_q_heads=48, n_kv_heads=6, seed=44)
    dp = DevProblem(p)
    ctx = make_ctx(p)
    full = to_bits(run(ctx, dp))
    pw = synth.make_problem(name="sched_48_6_window", T=4096, n_q_heads=48, n_kv_heads=6, seed=44, q_base=1024)
    win = to_bits(run(ctx, DevProblem(pw)))
    ctx.close()
    rows = sample_rows(p.rows, k=16, seed=5)
    rec = parity_record("48/6 table", full[rows], oracle_rows(orc, p, rows), p.n_q_heads, rows)
    say(f"  {rec}")
    check_parity(rec)
    assert np.array_equal(win, full[1024:]), "window rows differ from the full pass"
    out = torch.empty((p.T, p.n_q_heads * 256), dtype=torch.bfloat16, device="cuda")
    geom = ga.geometry(p.n_q_heads, p.n_kv_heads, p.T, p.rms_eps)
    inp = ga.attn_inputs(dp.qg.data_ptr(), dp.k.data_ptr(), dp.v.data_ptr(), dp.wq.data_ptr(), dp.wk.data_ptr(),
                         dp.cos.data_ptr(), dp.sin.data_ptr(), dp.cos.shape[0])
    assert ga.attn_prefill_gated_noalloc(geom, inp, p.T, out.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream) == ga.ATTN_OK
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), full), "table and snake passes differ"


# --------------------------------------------------------------------------
# The workloads at full size, in the benchmark's launch configuration,
# on sampled rows the oracle computes one by one
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_parity_configs_sampled(orc, name):
    say(f"config {name}")
    p = cfg(name)
    got = gpu_out(p)
    rows = sample_rows(p.rows, k=24 if p.T > 4096 else 64, seed=1)
    want = oracle_rows(orc, p, rows)
    rec = parity_record(f"config {name}", got[rows], want, p.n_q_heads, rows)
    say(f"  {rec}")
    check_parity(rec)
    assert np.isfinite(bits_to_f32(got)).all()


# --------------------------------------------------------------------------
# Bit-exact identities on the GPU
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,qb,Hq,Hkv", [(700, 128, 24, 2), (2048, 1024, 16, 4), (8192, 1024, 24, 2)])
def test_prefix_window_equals_full_pass(T, qb, Hq, Hkv):
    say(f"prefix==full T={T} q_base={qb}")
    full = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=21)
    win = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, q_base=qb, seed=21)
    ctx = make_ctx(full)
    a = gpu_out(full, ctx)
    b = gpu_out(win, ctx)
    ctx.close()
    assert np.array_equal(a[qb:], b)


@pytest.mark.parametrize("T,Hq,Hkv", [(300, 24, 2), (2048, 16, 4)])
def test_bidirectional_last_row_equals_causal(T, Hq, Hkv):
    """The last row sees every key in both passes: the same row bit for bit; the
    first row differs (it sees later keys only in the bidirectional pass)."""
    say(f"bidirectional last row T={T}")
    pc = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=25)
    pb = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=25, causal=False)
    ctx = make_ctx(pc)
    a = gpu_out(pc, ctx)
    b = gpu_out(pb, ctx)
    ctx.close()
    assert np.array_equal(a[-1], b[-1])
    assert not np.array_equal(a[0], b[0])


@pytest.mark.parametrize("T,chunks,Hq,Hkv", [(700, [256, 512], 24, 2), (8192, [1024, 4096], 16, 4)])
def test_append_chunks_equal_full_pass(T, chunks, Hq, Hkv):
    """Appending chunks to a K/V cache (prepared keys kept from earlier calls)
    reproduces the full pass's rows bit for bit."""
    say(f"append chunks T={T} at {chunks}")
    full = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=26)
    ctx = make_ctx(full)
    want = gpu_out(full, ctx)
    dp = DevProblem(full)
    cache = ctx.kv_cache()
    bounds = [0] + list(chunks) + [T]
    outs = [ctx.prefill_append(dp.qg[a:b], dp.k[a:b], dp.v[a:b], dp.wq, dp.wk, dp.cos, dp.sin, b, a, cache)
            for a, b in zip(bounds[:-1], bounds[1:])]
    torch.cuda.synchronize()
    got = to_bits(torch.cat(outs))
    ctx.close()
    assert np.array_equal(got, want)


def test_branches_continue_a_shared_prefix_cache():
    """Branches continued from one prefix cache (each call prepares its own new
    keys over the previous branch's) give, bit for bit, one pass over prefix +
    branch, in any order and repeated; bf16 and fp8 caches."""
    P, lens, Hq, Hkv = 256, [1, 200, 37, 128], 16, 4
    Tmax = P + max(lens)
    say(f"shared prefix P={P} branches {lens}")
    A = synth.make_problem(T=Tmax, n_q_heads=Hq, n_kv_heads=Hkv, seed=50)
    da = DevProblem(A)
    dbs = [DevProblem(synth.make_problem(T=Tmax, n_q_heads=Hq, n_kv_heads=Hkv, seed=60 + i))
           for i in range(len(lens))]
    ctx = make_ctx(A)

    def tokens(i):
        T = P + lens[i]
        cat = lambda x, y: torch.cat([x[:P], y[P:T]]).contiguous()
        return cat(da.qg, dbs[i].qg), cat(da.k, dbs[i].k), cat(da.v, dbs[i].v), T

    for fp8 in (False, True):
        want = []
        for i in range(len(lens)):
            qg, k, v, T = tokens(i)
            if fp8:
                fresh = ctx.kv_cache_fp8()
                full = ctx.prefill_append_fp8(qg, k, v, da.wq, da.wk, da.cos, da.sin, T, 0, fresh)
            else:
                full = ctx.prefill_gated(qg, k, v, da.wq, da.wk, da.cos, da.sin)
            want.append(to_bits(full)[P:])
        cache = ctx.kv_cache_fp8() if fp8 else ctx.kv_cache()
        append = ctx.prefill_append_fp8 if fp8 else ctx.prefill_append
        append(da.qg[:P], da.k[:P], da.v[:P], da.wq, da.wk, da.cos, da.sin, P, 0, cache)
        for i in [2, 0, 3, 1, 2, 0]:
            qg, k, v, T = tokens(i)
            got = to_bits(append(qg[P:], k[P:], v[P:], da.wq, da.wk, da.cos, da.sin, T, P, cache))
            assert np.array_equal(got, want[i]), f"branch {i} (fp8={fp8})"
    ctx.close()


def test_append_window_vs_oracle(orc):
    """The last appended chunk against the oracle's prefix window."""
    say("append window vs oracle")
    T, qb = 650, 512
    full = synth.make_problem(T=T, n_q_heads=8, n_kv_heads=2, seed=27)
    win = synth.make_problem(T=T, n_q_heads=8, n_kv_heads=2, q_base=qb, seed=27)
    ctx = make_ctx(full)
    dp = DevProblem(full)
    cache = ctx.kv_cache()
    ctx.prefill_append(dp.qg[:qb], dp.k[:qb], dp.v[:qb], dp.wq, dp.wk, dp.cos, dp.sin, qb, 0, cache)
    out = ctx.prefill_append(dp.qg[qb:], dp.k[qb:], dp.v[qb:], dp.wq, dp.wk, dp.cos, dp.sin, T, qb, cache)
    torch.cuda.synchronize()
    got = to_bits(out)
    ctx.close()
    rec = parity_record("append window t650 qb512", got, orc.attention(win, threads=8), win.n_q_heads)
    say(f"  {rec}")
    check_parity(rec)


@pytest.mark.parametrize("T", [300, 2048])
def test_all_visible_mask_equals_dense(T):
    say(f"mask all visible T={T}")
    p = synth.make_problem(T=T, seed=22)
    pm = synth.Problem(**{**p.__dict__, "mask": np.full((T, T), 3, np.uint8)})
    ctx = make_ctx(p)
    assert np.array_equal(gpu_out(p, ctx), gpu_out(pm, ctx))
    ctx.close()


def test_gqa_copy_equals_grouped():
    say("gqa copy")
    p = synth.make_problem(T=260, n_q_heads=12, n_kv_heads=2, seed=23)
    p12 = synth.Problem(**{**p.__dict__, "n_kv_heads": 12, "k": np.repeat(p.k, 6, axis=1),
                           "v": np.repeat(p.v, 6, axis=1)})
    assert np.array_equal(gpu_out(p), gpu_out(p12))


def test_gate_closed_forms(orc):
    """Gate logit 32 gives sigmoid 1 (out = ctx); logit 0 gives 1/2 (out = ctx / 2, exact)."""
    say("gate closed forms")
    p = synth.make_problem(T=150, n_q_heads=8, n_kv_heads=2, seed=24)
    outs = {}
    for gv in [0.0, 32.0]:
        q = p.qg.copy()
        q[:, :, 1, :] = synth.f32_to_bf16_bits(np.full(1, gv, np.float32))[0]
        outs[gv] = bits_to_f32(gpu_out(synth.Problem(**{**p.__dict__, "qg": q})))
    assert np.array_equal(outs[0.0] * 2, outs[32.0])
    # and the saturated output is the ungated context within the tolerance
    ctx_ref = orc.attention(p, want_ctx=True)["ctx"]
    bad, _ = parity_report(synth.f32_to_bf16_bits(outs[32.0]), ctx_ref)
    assert bad == 0


@pytest.mark.parametrize("masked", [False, True])
def test_one_hot_v_zero_pattern(masked):
    """One-hot V and a saturated gate expose each key's weight: hidden keys give
    exactly +0, visible keys a positive weight; repeated over 256-key windows."""
    T, Hq, Hkv = 512, 8, 2
    say(f"one-hot masked={masked}")
    p = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=25,
                           mask_budget=37 if masked else None)
    v = np.zeros((T, Hkv, 256), np.float32)
    for j in range(T):
        v[j, :, j % 256] = 1.0
    q = p.qg.copy()
    q[:, :, 1, :] = synth.f32_to_bf16_bits(np.full(1, 32.0, np.float32))[0]
    pp = synth.Problem(**{**p.__dict__, "qg": q, "v": synth.f32_to_bf16_bits(v)})
    got = bits_to_f32(gpu_out(pp)).reshape(T, Hq, 256)
    vis = np.tril(np.ones((T, T), bool))
    if pp.mask is not None:
        vis &= pp.mask != 0
    for i in range(T):
        # weights fold onto dims j % 256; rows < 256 see each dim at most once
        if i >= 256:
            break
        want_nz = vis[i, :256]
        g = got[i]
        assert np.all(g[:, ~want_nz] == 0.0), f"row {i}: hidden key leaked"
        assert np.all(g[:, want_nz] > 0.0), f"row {i}: visible key dropped"
        assert not np.signbit(g).any()
    # keys 256..511 fold onto the same dims; rows >= 256: dim d carries keys d and d+256
    for i in range(256, T, 17):
        both = vis[i, :256] | vis[i, 256:512]
        g = got[i]
        assert np.all(g[:, ~both] == 0.0) and np.all(g[:, both] > 0.0), f"row {i}"


def _visible_rows(p, rows, k0, k1, dev):
    """[len(rows)][k1-k0] visibility of keys k0..k1-1, from its definition: causal on
    absolute positions, ANDed with the mask (non-zero = visible) where there is one."""
    rows_t = torch.as_tensor(np.asarray(rows), device=dev)
    keys = torch.arange(k0, k1, device=dev)
    vis = keys[None, :] <= (p.q_base + rows_t)[:, None]
    return vis


@pytest.mark.parametrize("name", ["c2_dense_s8192_g4", "c4_masked_s8192"])
def test_one_hot_v_windows_full_size(name):
    """The full-size zero-pattern check: for each of the 8192 / 256 = 32 windows of
    256 keys, V is one-hot over the window (key 256w + d carries e_d at every KV
    head, every other key zero) and the gate saturated (logit 32: bf16(sigmoid) is
    exactly 1), so output element (i, h, d) is key 256w + d's weight for row i.
    Every hidden key (past the row, or masked) must give exactly +0 and every
    visible key a positive value, for every row, head and window (the QSA kernel
    page, "Validation": the controls; "Semantics": non-zero = visible)."""
    p = cfg(name)
    say(f"one-hot V over 256-key windows, {name}")
    dp = DevProblem(p)
    Hq, T = p.n_q_heads, p.T
    dp.qg.view(p.rows, Hq, 2, 256)[:, :, 1, :] = 32.0
    ctx = make_ctx(p)
    out = torch.empty((p.rows, Hq * 256), dtype=torch.bfloat16, device="cuda")
    ar = torch.arange(256, device="cuda")
    rows = np.arange(p.rows)
    hidden_nz = visible_zero = negative = 0
    for w in range(T // 256):
        v = torch.zeros_like(dp.v)
        v[256 * w + ar, :, ar] = 1.0
        dp.v = v
        run(ctx, dp, out=out)
        o = out.view(p.rows, Hq, 256)
        vis = _visible_rows(p, rows, 256 * w, 256 * w + 256, "cuda")
        if dp.mask is not None:
            vis &= dp.mask[:, 256 * w:256 * w + 256] != 0
        nz = o != 0
        hidden_nz += int((nz & ~vis[:, None, :]).sum())
        visible_zero += int((~nz & vis[:, None, :]).sum())
        negative += int(torch.signbit(o).sum())
    torch.cuda.synchronize()
    ctx.close()
    say(f"  hidden keys with a non-zero weight: {hidden_nz}; visible keys at zero: {visible_zero}; "
        f"negative or -0: {negative}")
    assert hidden_nz == 0 and visible_zero == 0 and negative == 0


def _perturbed(dp, hidden_keys, seed):
    """Copies of dp's K and V with the rows of `hidden_keys` (bool [T] on the
    device) replaced by fresh N(0, 4) values."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    k, v = dp.k.clone(), dp.v.clone()
    n = int(hidden_keys.sum())
    if n:
        k[hidden_keys] = (2.0 * torch.randn((n,) + tuple(k.shape[1:]), device="cuda", generator=g)).to(k.dtype)
        v[hidden_keys] = (2.0 * torch.randn((n,) + tuple(v.shape[1:]), device="cuda", generator=g)).to(v.dtype)
    return k, v


@pytest.mark.parametrize("name,rows", [("c4_masked_s8192", [0, 63, 2047, 2048, 3001, 4095, 6143, 8191]),
                                       ("c2_dense_s8192_g4", [0, 31, 32, 1000, 4095, 8190])])
def test_hidden_keys_perturbation_invariance_per_row(name, rows):
    """Row by row: randomising the K and V rows of every key hidden from row i (past
    it, or masked) leaves row i's output bit-identical, whatever those keys hold
    (their scores are -inf for that row and their weights exactly 0), while the
    other rows change.  At the masked workload's density (2048 of up to 8192 keys
    per row) almost no key is hidden from all 64 rows of a row block, so the per-row
    form is the one that reaches the mask bits; the block form follows."""
    p = cfg(name)
    say(f"perturbation invariance per row, {name}")
    dp = DevProblem(p)
    ctx = make_ctx(p)
    base = run(ctx, dp).clone()
    for i in rows:
        hid = ~_visible_rows(p, [i], 0, p.T, "cuda")[0]
        if dp.mask is not None:
            hid |= dp.mask[i] == 0
        dk = DevProblem.__new__(DevProblem)
        dk.__dict__.update(dp.__dict__)
        dk.k, dk.v = _perturbed(dp, hid, seed=1000 + i)
        got = run(ctx, dk)
        torch.cuda.synchronize()
        n_hidden = int(hid.sum())
        same = torch.equal(got[i], base[i])
        changed = int((got != base).any(dim=1).sum())
        say(f"  row {i}: {n_hidden} hidden keys perturbed; row identical={same}; rows changed={changed}")
        assert same
        if n_hidden:
            assert changed > 0                       # the perturbation reached the pass
    ctx.close()


def test_hidden_keys_perturbation_invariance_per_block(orc):
    """Per 64-row block of the masked workload: with the block's mask rows cleared on
    a random half of its 32-key tiles and a random quarter of the other keys, the
    keys hidden from all 64 rows (those, plus the block's causal future) are
    randomised in K and V; the block's 64 rows stay bit-identical.  The cleared
    tiles are skipped by the walk (no copy, no product), so this covers the
    tile-skip path as well as the per-key hide; sampled rows of each block also
    match the oracle (a walk over the wrong visible tiles would be invariant
    too, but not equal to it)."""
    p = cfg("c4_masked_s8192")
    say("perturbation invariance per block, c4 with cleared tiles")
    rng = np.random.default_rng(7)
    mask = np.array(p.mask, copy=True)
    blocks = [32, 64, 127]                           # rows 2048.., 4096.., 8128..
    for rb in blocks:
        r0 = 64 * rb
        ntile = (r0 + 64) // 32
        tiles = np.nonzero(rng.random(ntile) < 0.5)[0]
        cols = (32 * tiles[:, None] + np.arange(32)[None, :]).ravel()
        cols = np.concatenate([cols, np.nonzero(rng.random(r0 + 64) < 0.25)[0]])
        mask[r0:r0 + 64, cols] = 0
    pm = synth.Problem(**{**p.__dict__, "mask": mask})
    dp = DevProblem(pm)
    ctx = make_ctx(pm)
    base = run(ctx, dp).clone()
    rows = np.array([64 * rb + r for rb in blocks for r in (0, 17, 40, 63)], dtype=np.int32)
    rec = parity_record("c4 cleared tiles", to_bits(base)[rows], oracle_rows(orc, pm, rows), pm.n_q_heads, rows)
    say(f"  {rec}")
    check_parity(rec)
    for rb in blocks:
        r0 = 64 * rb
        vis = (dp.mask[r0:r0 + 64] != 0) & _visible_rows(pm, np.arange(r0, r0 + 64), 0, pm.T, "cuda")
        hid = ~vis.any(dim=0)
        dk = DevProblem.__new__(DevProblem)
        dk.__dict__.update(dp.__dict__)
        dk.k, dk.v = _perturbed(dp, hid, seed=rb)
        got = run(ctx, dk)
        torch.cuda.synchronize()
        n_before = int(hid[:r0 + 64].sum())
        same = torch.equal(got[r0:r0 + 64], base[r0:r0 + 64])
        say(f"  block {rb}: {n_before} keys at or before its last row hidden from all its rows "
            f"(of {r0 + 64}); rows identical={same}")
        assert n_before > (r0 + 64) // 3               # a real share of the block's keys is hidden
        assert same
    ctx.close()


def test_row_sums_at_max_tokens():
    """At the library's token cap (32768 keys) with V = 1 and the gate saturated, the
    output is the sum of the row's weights: 1 within 2e-3 (the QSA kernel page's
    review, item F2: row sums at exactly the token cap), for every row and head; the
    walk covers every visible key up to the last row."""
    import gated_gqa_causal_amd as ga
    T = ga.ATTN_MAX_TOKENS
    say(f"row sums at {T}")
    p = synth.make_problem(T=T, n_q_heads=4, n_kv_heads=1, seed=26)
    q = p.qg.copy()
    q[:, :, 1, :] = synth.f32_to_bf16_bits(np.full(1, 32.0, np.float32))[0]
    pp = synth.Problem(**{**p.__dict__, "qg": q, "v": np.full_like(p.v, 0x3F80)})
    ctx = ga.Context(4, 1, T)
    got = bits_to_f32(gpu_out(pp, ctx))
    ctx.close()
    worst = float(np.abs(got - 1.0).max())
    say(f"  max |row sum - 1| = {worst:.3g}")
    assert worst <= 2e-3


def test_library_max_tokens(orc):
    """At the library's token cap: sampled rows against the oracle (row and key
    offsets at their largest), and the last 1024 rows as a prefix window equal
    to the full pass's rows bit for bit."""
    import gated_gqa_causal_amd as ga
    T = ga.ATTN_MAX_TOKENS
    say(f"library max tokens T={T}, 4/1 heads")
    p = synth.make_problem(T=T, n_q_heads=4, n_kv_heads=1, seed=41)
    ctx = ga.Context(4, 1, T)
    got = gpu_out(p, ctx)
    rows = sample_rows(p.rows, k=16, seed=3)
    want = oracle_rows(orc, p, rows)
    rec = parity_record(f"cap {T} dense", got[rows], want, p.n_q_heads, rows)
    say(f"  {rec}")
    check_parity(rec)
    assert np.isfinite(bits_to_f32(got)).all()
    pw = synth.make_problem(T=T, n_q_heads=4, n_kv_heads=1, seed=41, q_base=T - 1024)
    win = gpu_out(pw, ctx)
    ctx.close()
    assert np.array_equal(win, got[T - 1024:])


def test_masked_library_max_tokens(orc):
    """Masked pass at the token cap: a [32768][32768] u8 mask (each key visible
    with probability 1/4, causality ANDed by the pass), so the longest row
    block's tile list holds every one of its 1024 key tiles; sampled rows
    against the oracle."""
    import gated_gqa_causal_amd as ga
    T = ga.ATTN_MAX_TOKENS
    say(f"masked library max tokens T={T}, 4/1 heads")
    p = synth.make_problem(T=T, n_q_heads=4, n_kv_heads=1, seed=42)
    rng = np.random.default_rng(42)
    mask = np.empty((T, T), dtype=np.uint8)
    for r0 in range(0, T, 2048):
        mask[r0:r0 + 2048] = rng.integers(0, 4, size=(2048, T), dtype=np.uint8) == 0
    pm = synth.Problem(**{**p.__dict__, "mask": mask})
    got = gpu_out(pm)
    rows = sample_rows(pm.rows, k=16, seed=4)
    want = oracle_rows(orc, pm, rows)
    rec = parity_record(f"cap {T} masked", got[rows], want, pm.n_q_heads, rows)
    say(f"  {rec}")
    check_parity(rec)
    assert np.isfinite(bits_to_f32(got)).all()


# --------------------------------------------------------------------------
# Negative controls: the gate is not vacuous
# --------------------------------------------------------------------------

def test_control_kv_head_swap_fails(orc):
    say("control: kv swap")
    p = synth.make_problem(T=200, n_q_heads=24, n_kv_heads=2, seed=27)
    swapped = synth.Problem(**{**p.__dict__, "k": p.k[:, ::-1].copy(), "v": p.v[:, ::-1].copy()})
    got, want = gpu_out(swapped), orc.attention(p, threads=8)
    bad, _ = parity_report(got, want)
    assert bad > 0
    with pytest.raises(AssertionError):
        check_parity(parity_record("control kv swap", got, want, p.n_q_heads))


def test_control_causal_for_mask_fails(orc):
    say("control: causal in place of the mask")
    p = synth.make_problem(T=600, n_q_heads=8, n_kv_heads=2, seed=28, mask_budget=64)
    dense = synth.Problem(**{**p.__dict__, "mask": None})
    rows = np.arange(300, 600, 7, dtype=np.int32)
    got, want = gpu_out(dense)[rows], orc.attention(p, rows=rows, threads=8)
    bad, _ = parity_report(got, want)
    assert bad > 0
    with pytest.raises(AssertionError):
        check_parity(parity_record("control causal for mask", got, want, p.n_q_heads))


# --------------------------------------------------------------------------
# Edges of the boundary on a real device
# --------------------------------------------------------------------------

def test_empty_and_refusals_on_device():
    import gated_gqa_causal_amd as ga
    say("edges")
    p = synth.make_problem(T=256, n_q_heads=4, n_kv_heads=2, seed=29)
    ctx = make_ctx(p)
    dp = DevProblem(p)
    inp = ctx.inputs(*dp.args(), 256, 256)
    out = torch.empty((256, 4 * 256), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert ga.attn_prefill_gated(ctx.handle, inp, 0, None, s) == ga.ATTN_OK
    assert ga.attn_prefill_prefix(ctx.handle, inp, 256, 256, None, s) == ga.ATTN_OK
    assert ga.attn_prefill_prefix(ctx.handle, inp, 256, 64, out.data_ptr(), s) == ga.ATTN_ERR_ALIGN
    assert ga.attn_prefill_gated(ctx.handle, inp, 257, out.data_ptr(), s) == ga.ATTN_ERR_RANGE
    assert ga.attn_prefill_masked(ctx.handle, inp, 256, None, out.data_ptr(), s) == ga.ATTN_ERR_NULL_ARG
    torch.cuda.synchronize()
    ctx.close()


def test_timing_hooks():
    import gated_gqa_causal_amd as ga
    p = synth.make_problem(T=512, n_q_heads=8, n_kv_heads=2, seed=30)
    ctx = make_ctx(p)
    dp = DevProblem(p)
    ctx.set_timing(True)
    for _ in range(3):
        run(ctx, dp)
    ms, n = ctx.read_timing(ga.ATTN_KERNEL_ATTENTION)
    assert n == 3 and ms > 0
    ms, n = ctx.read_timing(ga.ATTN_KERNEL_KV_PROLOGUE)
    assert n == 3 and ms > 0
    # Only the attention kernel's launches.
    ctx.set_timing(True, kernels=[ga.ATTN_KERNEL_ATTENTION])
    for _ in range(2):
        run(ctx, dp)
    assert ctx.read_timing(ga.ATTN_KERNEL_KV_PROLOGUE) == (0.0, 0)
    ms, n = ctx.read_timing(ga.ATTN_KERNEL_ATTENTION)
    assert n == 2 and ms > 0
    assert ga.attn_ctx_set_timing_mask(ctx.handle, ga.ATTN_TIMING_ALL + 1) == ga.ATTN_ERR_RANGE
    ctx.set_timing(False)
    ctx.close()


@pytest.mark.gpu
def test_mfma_clock_probe_is_plausible():
    """The calibration kernel runs and reports a clock and rate a gfx950 can
    have: at most the 2.4 GHz boost clock and the matching 2.5 PFLOP/s."""
    import gated_gqa_causal_amd as ga
    say("mfma clock probe")
    mhz, tf = ga.attn_mfma_clock_probe(2000)
    assert 300.0 < mhz < 2500.0
    assert 100.0 < tf < 2600.0
    # rate and clock agree: 4 SIMDs x 1024 FLOP per cycle per compute unit
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert abs(tf * 1e12 / (cus * 4 * 1024 * mhz * 1e6) - 1.0) < 0.1


# --------------------------------------------------------------------------
# Packed batches: each sequence gets the bits it gets alone
# --------------------------------------------------------------------------

def _batch_tensors(b):
    from gpu_util import bf16_tensor
    s0 = b.seqs[0]
    return dict(qg=bf16_tensor(b.qg), k=bf16_tensor(b.k), v=bf16_tensor(b.v), wq=bf16_tensor(s0.q_norm_w),
                wk=bf16_tensor(s0.k_norm_w), cos=torch.from_numpy(np.ascontiguousarray(s0.cos)).to("cuda"),
                sin=torch.from_numpy(np.ascontiguousarray(s0.sin)).to("cuda"))


def _batch_call(ctx, b, t):
    return ctx.prefill_gated_batch(t["qg"], t["k"], t["v"], t["wq"], t["wk"], t["cos"], t["sin"], b.lens)


def _batch_out(b):
    import gated_gqa_causal_amd as ga
    s0 = b.seqs[0]
    # each sequence's keys start on a 32-key tile of the workspace
    ctx = ga.Context(s0.n_q_heads, s0.n_kv_heads, max(sum((L + 31) // 32 * 32 for L in b.lens), 1), s0.rms_eps)
    out = _batch_call(ctx, b, _batch_tensors(b))
    torch.cuda.synchronize()
    res = to_bits(out)
    ctx.close()
    return res


def _offsets(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(int)


@pytest.mark.parametrize("lens,Hq,Hkv", [([1, 31, 32, 33, 0, 64, 65, 200, 130], 24, 2),
                                         ([300, 7, 128], 16, 4), ([5], 6, 1), ([0, 0, 97, 0], 2, 2)])
def test_batch_equals_sequences_alone(lens, Hq, Hkv):
    say(f"batch {lens} {Hq}/{Hkv}")
    b = synth.make_batch(lens, n_q_heads=Hq, n_kv_heads=Hkv, seed=len(lens))
    got = _batch_out(b)
    off = _offsets(lens)
    for i, p in enumerate(b.seqs):
        if p.T == 0:
            continue
        alone = gpu_out(p)
        assert np.array_equal(got[off[i]:off[i + 1]], alone), f"sequence {i} (len {p.T}) differs"


@pytest.mark.parametrize("T,Hq,Hkv,q_base", [(2048, 24, 2, 0), (64, 24, 2, 0), (1000, 16, 4, 0), (8192, 24, 2, 7680),
                                             (2085, 8, 8, 0), (3072, 24, 2, 0), (4096, 16, 4, 0),
                                             (8192, 24, 2, 5120)])
def test_split_items_equal_whole_items(T, Hq, Hkv, q_base):
    """Launches with few work items per compute unit split their heaviest
    items into 32-row halves, each on one wave per SIMD, and deal the pieces
    over every compute unit, some taking several (the host table); a packed
    batch of the same one sequence never splits.  The rows agree bit for bit
    (a prefix window against the full pass's rows of the same sequence)."""
    say(f"split items T={T} {Hq}/{Hkv} q_base={q_base}")
    full = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=T + Hq)
    packed = _batch_out(synth.Batch(name="one", seqs=[full]))
    if q_base == 0:
        got = gpu_out(full)
        assert np.array_equal(got, packed)
    else:
        got = gpu_out(synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=T + Hq, q_base=q_base))
        assert np.array_equal(got, packed[q_base:])


@pytest.mark.parametrize("T,big,Hq,Hkv,budget", [(2048, 8192, 24, 2, 512), (1000, 8192, 32, 4, 300),
                                                  (64, 8192, 24, 2, 16), (3072, 8192, 24, 2, 768)])
def test_masked_split_items_equal_whole_items(T, big, Hq, Hkv, budget):
    """Masked: a T-key problem (few items per compute unit, so split) and the
    first T rows of a larger one with the same first T keys, rows and mask rows
    (enough items that nothing splits).  A row sees keys up to itself only, so
    the rows agree bit for bit."""
    say(f"masked split items T={T} (whole in a {big}-key pass) {Hq}/{Hkv} budget {budget}")
    pb = synth.make_problem(T=big, n_q_heads=Hq, n_kv_heads=Hkv, seed=T + Hq, mask_budget=budget)
    assert (big // 64) * -(-(Hq // Hkv) // 4) > 2 * (256 // Hkv)     # whole items only (items a KV head > 2 P / Hkv)
    ps = synth.Problem(**{**pb.__dict__, "T": T, "qg": pb.qg[:T], "k": pb.k[:T], "v": pb.v[:T],
                          "cos": pb.cos[:T], "sin": pb.sin[:T], "mask": np.ascontiguousarray(pb.mask[:T, :T])})
    assert np.array_equal(gpu_out(ps), gpu_out(pb)[:T])


def test_batch_order_does_not_matter():
    lens = [200, 33, 0, 130, 64]
    b = synth.make_batch(lens, n_q_heads=8, n_kv_heads=2, seed=11)
    got = _batch_out(b)
    perm = [3, 0, 4, 2, 1]
    bp = synth.Batch(name="perm", seqs=[b.seqs[i] for i in perm])
    gotp = _batch_out(bp)
    off, offp = _offsets(lens), _offsets([lens[i] for i in perm])
    for jp, i in enumerate(perm):
        assert np.array_equal(got[off[i]:off[i + 1]], gotp[offp[jp]:offp[jp + 1]])


def test_batch_vs_oracle(orc):
    b = synth.make_batch([97, 1, 160, 33], n_q_heads=24, n_kv_heads=2, seed=21, gate_sigma=2.0)
    got = _batch_out(b)
    off = _offsets(b.lens)
    for i, p in enumerate(b.seqs):
        want = orc.attention(p, threads=8)
        rec = parity_record(f"batch seq {i} len {p.T}", got[off[i]:off[i + 1]], want, p.n_q_heads)
        say(f"  {rec}")
        check_parity(rec)


def test_batch_at_the_token_cap(orc):
    """The largest packed batch the cap admits: 1024 sequences of 1..32 tokens
    (each starts on a 32-key tile, 1024 x 32 = 32768 keys), 1024 row blocks
    in one launch, every sequence against the oracle."""
    import gated_gqa_causal_amd as ga
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(1, 33, size=ga.ATTN_MAX_TOKENS // 32)]
    lens[0], lens[-1] = 32, 1
    b = synth.make_batch(lens, n_q_heads=4, n_kv_heads=1, seed=23)
    say(f"batch at the cap: {len(lens)} sequences, {b.total} tokens")
    got = _batch_out(b)
    off = _offsets(b.lens)
    want = np.concatenate([orc.attention(p, threads=1) for p in b.seqs])
    rec = parity_record(f"batch at the cap ({len(lens)} sequences)", got, want, 4)
    say(f"  {rec}")
    check_parity(rec)
    assert np.isfinite(bits_to_f32(got)).all()


def test_batch_workload_sampled(orc):
    """The packed workload at full size: three sequences against their own
    launches bit for bit, sampled rows of three against the oracle."""
    b = synth.config_batch("c6_varlen_16x128_2048")
    say(f"batch workload {b.name} lens={b.lens}")
    got = _batch_out(b)
    off = _offsets(b.lens)
    order = np.argsort(b.lens)
    for i in [int(order[0]), int(order[len(order) // 2]), int(order[-1])]:
        p = b.seqs[i]
        assert np.array_equal(got[off[i]:off[i + 1]], gpu_out(p)), f"sequence {i}"
        rows = sample_rows(p.rows, k=16, seed=i)
        want = oracle_rows(orc, p, rows)
        rec = parity_record(f"batch workload seq {i} len {p.T}", got[off[i]:off[i + 1]][rows], want,
                            p.n_q_heads, rows)
        say(f"  {rec}")
        check_parity(rec)
    assert np.isfinite(bits_to_f32(got)).all()


def test_batch_reuses_context_back_to_back():
    """Two batches issued back to back on one context (the staging buffer is
    reused) both give their sequences' bits."""
    import gated_gqa_causal_amd as ga
    b1 = synth.make_batch([64, 200], n_q_heads=8, n_kv_heads=2, seed=31)
    b2 = synth.make_batch([130, 7, 96], n_q_heads=8, n_kv_heads=2, seed=32)
    ctx = ga.Context(8, 2, 512, 1e-6)
    o1 = _batch_call(ctx, b1, _batch_tensors(b1))
    o2 = _batch_call(ctx, b2, _batch_tensors(b2))
    torch.cuda.synchronize()
    for b, o in ((b1, o1), (b2, o2)):
        off = _offsets(b.lens)
        got = to_bits(o)
        for i, p in enumerate(b.seqs):
            assert np.array_equal(got[off[i]:off[i + 1]], gpu_out(p))
    ctx.close()


# --------------------------------------------------------------------------
# Branches of one shared prefix in one launch
# --------------------------------------------------------------------------

def _shared_ctx(sp):
    """A context holding the prefix plus the longest branch (positions) and every
    branch's own keys on 32-key tiles (workspace)."""
    import gated_gqa_causal_amd as ga
    pre = sp.prefix
    need = max([sp.P + max(sp.lens + [0]), sum((L + 31) // 32 * 32 for L in sp.lens), 1])
    return ga.Context(pre.n_q_heads, pre.n_kv_heads, need, pre.rms_eps)


def _shared_run(sp, ctx=None):
    """The prefix appended to a fresh cache, then every branch through one
    attn_prefill_shared_batch call; (output bits, cache, context)."""
    from gpu_util import bf16_tensor
    own = ctx is None
    ctx = ctx or _shared_ctx(sp)
    pre = sp.prefix
    wq, wk = bf16_tensor(pre.q_norm_w), bf16_tensor(pre.k_norm_w)
    cos = torch.from_numpy(np.ascontiguousarray(pre.cos)).to("cuda")
    sin = torch.from_numpy(np.ascontiguousarray(pre.sin)).to("cuda")
    cache = ctx.kv_cache()
    if sp.P:
        ctx.prefill_append(bf16_tensor(pre.qg), bf16_tensor(pre.k), bf16_tensor(pre.v), wq, wk, cos, sin, sp.P, 0,
                           cache)
    out = ctx.prefill_shared_batch(bf16_tensor(sp.qg), bf16_tensor(sp.k), bf16_tensor(sp.v), wq, wk, cos, sin,
                                   sp.P, cache if sp.P else None, sp.lens)
    torch.cuda.synchronize()
    got = to_bits(out)
    if own:
        ctx.close()
        return got, None, None
    return got, cache, ctx


@pytest.mark.parametrize("P,lens,Hq,Hkv", [(128, [1, 31, 32, 33, 0, 64, 65, 200, 130], 24, 2),
                                           (1024, [300, 7, 128], 16, 4), (256, [5], 6, 1),
                                           (384, [0, 0, 97, 0], 2, 2), (2048, [64] * 12 + [1, 190], 8, 8)])
def test_shared_batch_equals_branches_alone(P, lens, Hq, Hkv):
    """Each branch of one launch gets, bit for bit, the rows of its own prefix
    window over prefix + branch (the full pass's rows P..)."""
    say(f"shared prefix P={P} branches {lens} {Hq}/{Hkv}")
    sp = synth.make_shared_prefix(P, lens, n_q_heads=Hq, n_kv_heads=Hkv, seed=P + len(lens))
    got, _, _ = _shared_run(sp)
    off = _offsets(lens)
    for i, b in enumerate(sp.branches):
        if b.rows == 0:
            continue
        assert np.array_equal(got[off[i]:off[i + 1]], gpu_out(b)), f"branch {i} (len {b.rows}) differs"


def test_shared_batch_equals_appends_and_leaves_the_cache():
    """The same branches continued one call each from the cache (each append
    over a copy of it) give the launch's bits; the launch does not write the
    cache, and a second launch on the same context gives the same bits."""
    from gpu_util import bf16_tensor
    P, lens = 512, [200, 1, 37, 128]
    say(f"shared prefix vs appends P={P} {lens}")
    sp = synth.make_shared_prefix(P, lens, n_q_heads=16, n_kv_heads=4, seed=77)
    ctx = _shared_ctx(sp)
    got, cache, ctx = _shared_run(sp, ctx)
    before = cache.clone()
    pre = sp.prefix
    wq, wk = bf16_tensor(pre.q_norm_w), bf16_tensor(pre.k_norm_w)
    cos = torch.from_numpy(np.ascontiguousarray(pre.cos)).to("cuda")
    sin = torch.from_numpy(np.ascontiguousarray(pre.sin)).to("cuda")
    again = ctx.prefill_shared_batch(bf16_tensor(sp.qg), bf16_tensor(sp.k), bf16_tensor(sp.v), wq, wk, cos, sin,
                                     P, cache, lens)
    torch.cuda.synchronize()
    assert torch.equal(cache, before), "the shared launch wrote the prefix cache"
    assert np.array_equal(to_bits(again), got)
    off = _offsets(lens)
    for i, b in enumerate(sp.branches):
        c = before.clone()
        o = ctx.prefill_append(bf16_tensor(b.qg), bf16_tensor(b.k[P:]), bf16_tensor(b.v[P:]), wq, wk, cos, sin,
                               b.T, P, c)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(o), got[off[i]:off[i + 1]]), f"branch {i}"
    ctx.close()


def test_shared_batch_without_prefix_is_a_packed_batch():
    lens = [1, 31, 32, 33, 0, 64, 65, 200, 130]
    sp = synth.make_shared_prefix(0, lens, n_q_heads=24, n_kv_heads=2, seed=9)
    b = synth.make_batch(lens, n_q_heads=24, n_kv_heads=2, seed=9)
    got, _, _ = _shared_run(sp)
    assert np.array_equal(got, _batch_out(b))


def test_shared_batch_order_does_not_matter():
    P, lens = 256, [200, 33, 0, 130, 64]
    sp = synth.make_shared_prefix(P, lens, n_q_heads=8, n_kv_heads=2, seed=12)
    got, _, _ = _shared_run(sp)
    perm = [3, 0, 4, 2, 1]
    spp = synth.SharedPrefix(name="perm", prefix=sp.prefix, branches=[sp.branches[i] for i in perm])
    gotp, _, _ = _shared_run(spp)
    off, offp = _offsets(lens), _offsets([lens[i] for i in perm])
    for jp, i in enumerate(perm):
        assert np.array_equal(got[off[i]:off[i + 1]], gotp[offp[jp]:offp[jp + 1]])


def test_shared_batch_vs_oracle(orc):
    sp = synth.make_shared_prefix(256, [97, 1, 160, 33], n_q_heads=24, n_kv_heads=2, seed=21, gate_sigma=2.0)
    got, _, _ = _shared_run(sp)
    off = _offsets(sp.lens)
    for i, b in enumerate(sp.branches):
        rec = parity_record(f"shared prefix 256 branch {i} len {b.rows}", got[off[i]:off[i + 1]],
                            orc.attention(b, threads=8), b.n_q_heads)
        say(f"  {rec}")
        check_parity(rec)


def _random_shared_cases(n=20, seed=77):
    """Seeded random shared-prefix launches: a prefix of 0..1536 tokens (a
    multiple of 128), 1..6 branches of 0..300 tokens, a GQA shape with G in 1..16."""
    rng = np.random.default_rng(seed)
    shapes = [(24, 2), (16, 4), (8, 8), (32, 2), (6, 1), (12, 3), (40, 5), (2, 2), (48, 6), (16, 1)]
    cases = []
    for i in range(n):
        P = 128 * int(rng.integers(0, 13))
        lens = [int(x) for x in rng.integers(0, 301, size=int(rng.integers(1, 7)))]
        Hq, Hkv = shapes[int(rng.integers(len(shapes)))]
        cases.append((f"s{i:02d}_P{P}_{Hq}x{Hkv}_n{len(lens)}", P, lens, Hq, Hkv, 500 + i))
    return cases


@pytest.mark.parametrize("case", _random_shared_cases(), ids=[c[0] for c in _random_shared_cases()])
def test_shared_batch_random(orc, case):
    """Every branch of a random launch bit for bit against its own window pass
    and, every row and head, against the oracle (a row-head over the row-scale
    bounds may meet them under the other reading of the score's dot product)."""
    name, P, lens, Hq, Hkv, sd = case
    say(f"shared prefix random {name}: lens {lens}")
    sp = synth.make_shared_prefix(P, lens, n_q_heads=Hq, n_kv_heads=Hkv, seed=sd)
    got, _, _ = _shared_run(sp)
    off = _offsets(lens)
    for i, b in enumerate(sp.branches):
        if b.rows == 0:
            continue
        mine = got[off[i]:off[i + 1]]
        assert np.array_equal(mine, gpu_out(b)), f"branch {i} (len {b.rows}) differs from its window pass"
        rec = check_parity_either_reading(orc, b, mine, f"shared random {name} branch {i}")
        if rec["other_reading_row_heads"]:
            say(f"  {rec}")


def test_shared_batch_at_the_token_cap(orc):
    """Branches reaching the library's token cap: a 30720-token prefix and four
    branches of up to 2048 tokens (positions to 32767), 4/1 heads; every branch
    bit for bit against its own window pass, sampled rows of the longest
    against the oracle."""
    import gated_gqa_causal_amd as ga
    T = ga.ATTN_MAX_TOKENS
    P, lens = T - 2048, [2048, 1, 1000, 2047]
    say(f"shared prefix at the cap: P={P} branches {lens}, 4/1 heads")
    sp = synth.make_shared_prefix(P, lens, n_q_heads=4, n_kv_heads=1, seed=43)
    ctx = ga.Context(4, 1, T)
    got, _, ctx = _shared_run(sp, ctx)
    off = _offsets(lens)
    for i, b in enumerate(sp.branches):
        assert np.array_equal(got[off[i]:off[i + 1]], gpu_out(b, ctx)), f"branch {i} (len {b.rows})"
    ctx.close()
    b = sp.branches[0]
    rows = sample_rows(b.rows, k=12, seed=5)
    rec = parity_record(f"shared prefix cap {T} branch 0", got[off[0]:off[1]][rows], oracle_rows(orc, b, rows),
                        b.n_q_heads, rows)
    say(f"  {rec}")
    check_parity(rec)


def test_shared_batch_workload_sampled(orc):
    """The measured workload (a 4096-token prefix, 16 branches of 128-512
    tokens, 24/2): every branch bit for bit against its own window pass, and
    sampled rows of three branches against the oracle."""
    sp = synth.config_shared("c8_shared_4096_16x128_512")
    say(f"shared workload P={sp.P} lens {sp.lens}")
    got, _, _ = _shared_run(sp)
    off = _offsets(sp.lens)
    for i, b in enumerate(sp.branches):
        assert np.array_equal(got[off[i]:off[i + 1]], gpu_out(b)), f"branch {i}"
    for i in (0, 7, 15):
        b = sp.branches[i]
        rows = sample_rows(b.rows, k=8, seed=i)
        rec = parity_record(f"c8 branch {i} sampled rows", got[off[i]:off[i + 1]][rows],
                            oracle_rows(orc, b, rows), b.n_q_heads)
        say(f"  {rec}")
        check_parity(rec)


# --------------------------------------------------------------------------
# fp8 (e4m3) K/V cache rows
# --------------------------------------------------------------------------

def _fp8_run(p, chunks, ctx=None):
    """Appends p's keys (p.q_base == 0: qg holds every row) in chunks ending at
    the listed positions to a fresh fp8 cache; returns (each chunk's output
    rows, the cache tensor, the context)."""
    import gated_gqa_causal_amd as ga
    dp = DevProblem(p)
    ctx = ctx or ga.Context(p.n_q_heads, p.n_kv_heads, p.T, p.rms_eps)
    cache = ctx.kv_cache_fp8()
    outs = []
    for a, b in zip([0] + chunks[:-1], chunks):
        outs.append(ctx.prefill_append_fp8(dp.qg[a:b], dp.k[a:b], dp.v[a:b], dp.wq, dp.wk, dp.cos, dp.sin,
                                           b, a, cache))
    torch.cuda.synchronize()
    return outs, cache, ctx


def _fp8_outputs(p, chunks):
    """Stacked outputs of the chunks (query rows 0..T-1; p.q_base must be 0)."""
    outs, cache, ctx = _fp8_run(p, chunks)
    got = to_bits(torch.cat(outs))
    return got, cache, ctx


@pytest.mark.parametrize("T,Hq,Hkv", [(300, 24, 2), (129, 16, 4)])
def test_fp8_cache_rows_bit_exact(orc, T, Hq, Hkv):
    """The cache the GPU writes holds exactly the oracle's e4m3 codes and scales."""
    from oracle import fp8
    say(f"fp8 cache rows T={T} {Hq}/{Hkv}")
    p = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=T + 1)
    _, cache, ctx = _fp8_outputs(p, [T])
    kc, vc, ks, vs = ctx.fp8_cache_views(cache)
    want = fp8.fp8_cache_kv(orc, p)
    assert np.array_equal(kc[:, :T].cpu().numpy(), want["k_codes"]), "key codes"
    assert np.array_equal(vc[:, :T].cpu().numpy(), want["v_codes"]), "value codes"
    assert np.array_equal(ks[:, :T].cpu().numpy().view(np.uint32), want["k_scales"].view(np.uint32)), "key scales"
    assert np.array_equal(vs[:, :T].cpu().numpy().view(np.uint32), want["v_scales"].view(np.uint32)), "value scales"
    ctx.close()


def _f32_neighbours(vals, k):
    """Every fp32 value within k ulps of each of vals (positive, finite)."""
    u = np.asarray(vals, dtype=np.float32).view(np.int32).astype(np.int64)
    off = np.arange(-k, k + 1, dtype=np.int64)
    return np.unique((u[:, None] + off[None, :]).clip(0, 0x7F7FFFFF).astype(np.int32)).view(np.float32)


def test_fp8_writer_encoder_against_oracle():
    """The cache writer's e4m3 encode (the hardware convert) gives the
    oracle's code for every fp32 value within 64 ulps of each e4m3 value and
    of each midpoint between neighbours (ties to even), for 2^21 random
    values, zeros of both signs and values just past 448 (the largest
    quotient a row's scale can give is 448 (1 + 2^-23)); with sc = 1 the
    writer's division returns x itself."""
    from oracle import fp8
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2
    anchors = np.concatenate([pos[1:], mids, [2.0 ** -10, 2.0 ** -11]])
    near = _f32_neighbours(anchors, 64)
    rng = np.random.default_rng(7)
    rnd = (rng.integers(0x3A000000, 0x43E00000, 1 << 21, dtype=np.int64).astype(np.int32)).view(np.float32)
    tiny = (rng.integers(0, 0x3A000000, 1 << 16, dtype=np.int64).astype(np.int32)).view(np.float32)
    x = np.concatenate([near, rnd, tiny, [0.0, 448.0]]).astype(np.float32)
    x = x[x <= np.float32(448.0 * (1 + 2.0 ** -21))]
    x = np.concatenate([x, -x]).astype(np.float32)
    say(f"fp8 writer encoder: {x.size} values")
    q, codes = debug_fp8_encode(x, np.ones_like(x))
    assert np.array_equal(q.view(np.uint32), x.view(np.uint32)), "division by 1"
    want = fp8.e4m3_encode(x)
    bad = np.nonzero(codes != want)[0]
    assert bad.size == 0, [(float(x[i]), int(codes[i]), int(want[i])) for i in bad[:8]]


def test_fp8_writer_division_against_ieee():
    """The writer's division (a correctly rounded reciprocal per row, then a
    multiply and two FMAs per value) equals fp32 division bit for bit over
    2^20 quotients at scales from 2^-49 to 2^119, including quotients near
    fp32 ties and each row maximum's own quotient near 448; its codes are the
    oracle's codes of the true quotients."""
    from oracle import fp8
    rng = np.random.default_rng(11)
    n = 1 << 20
    sc = (rng.integers(0, 1 << 23, n) | (rng.integers(127 - 49, 127 + 119, n) << 23)).astype(np.int32)
    sc = sc.view(np.float32)
    mode = rng.integers(0, 3, n)
    u = (rng.integers(0, 1 << 23, n) | (rng.integers(127 - 12, 127 + 9, n) << 23)).astype(np.int32)
    u = np.minimum(u.view(np.float32).astype(np.float64), 448.0)          # quotients up to 448
    e = np.floor(np.log2(u))
    u = np.where(mode == 1, u + 2.0 ** (e - 24), u)                       # near an fp32 tie of the quotient
    u = np.where(mode == 2, 448.0 * (1 + rng.integers(-8, 9, n) * 2.0 ** -24), u)
    x = (u * sc.astype(np.float64)).astype(np.float32)
    x = np.where(rng.random(n) < 0.5, -x, x).astype(np.float32)
    say(f"fp8 writer division: {n} quotients")
    q, codes = debug_fp8_encode(x, sc)
    want = (x / sc).astype(np.float32)
    bad = np.nonzero(q.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, [(float(x[i]), float(sc[i]), float(q[i]), float(want[i])) for i in bad[:8]]
    assert np.array_equal(codes, fp8.e4m3_encode(want))


def test_fp8_cache_rows_wide_range(orc):
    """Value rows at magnitudes from bf16 subnormals to 2^120 (both sides of
    the writer's 2^-40 switch between its two division routes), and rows
    holding a NaN, +-inf, only zeros, only -0 or one nonzero value: codes and
    scales equal the oracle's bit for bit (a NaN makes the row's amax NaN and
    its scale 1; an infinite amax makes the scale inf)."""
    from oracle import fp8
    T, Hq, Hkv = 160, 16, 4
    p = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=77)
    v = p.v.copy()                                                 # [T][Hkv][D] bf16 bits
    base = synth.bf16_bits_to_f32(v).astype(np.float64)
    exps = [-133, -126, -100, -60, -49, -42, -41, -40, -39, -30, -20, 0, 20, 60, 100, 120]
    specials = ["nan", "inf", "-inf", "zero", "negzero", "one", "subnormal"]
    kinds = exps + specials
    for t in range(T):
        for c in range(Hkv):
            kind = kinds[(t * Hkv + c) % len(kinds)]
            if isinstance(kind, int):
                v[t, c] = synth.f32_to_bf16_bits((base[t, c] * 2.0 ** kind).astype(np.float32))
            elif kind in ("zero", "negzero"):
                v[t, c] = 0 if kind == "zero" else 0x8000
            elif kind == "one":
                v[t, c] = 0
                v[t, c, (t * 7) % 256] = synth.f32_to_bf16_bits(np.array([base[t, c, 0] or 1.0], np.float32))[0]
            elif kind == "subnormal":
                v[t, c] = np.where(base[t, c] < 0, 0x8000, 0) | (np.arange(256) % 127 + 1)
            else:
                j = (t * 13) % 256
                v[t, c, j] = {"nan": 0x7FC0, "inf": 0x7F80, "-inf": 0xFF80}[kind]
    p.v = v.astype(np.uint16)
    say(f"fp8 cache rows over magnitudes and special rows T={T} {Hq}/{Hkv}")
    _, cache, ctx = _fp8_outputs(p, [T])
    kc, vc, ks, vs = ctx.fp8_cache_views(cache)
    want = fp8.fp8_cache_kv(orc, p)
    assert np.array_equal(kc[:, :T].cpu().numpy(), want["k_codes"]), "key codes"
    assert np.array_equal(ks[:, :T].cpu().numpy().view(np.uint32), want["k_scales"].view(np.uint32)), "key scales"
    got_vc, got_vs = vc[:, :T].cpu().numpy(), vs[:, :T].cpu().numpy()
    bad = np.argwhere((got_vc != want["v_codes"]).any(axis=-1)
                      | (got_vs.view(np.uint32) != want["v_scales"].view(np.uint32)))
    assert bad.size == 0, [(int(c), int(t), kinds[(int(t) * Hkv + int(c)) % len(kinds)]) for c, t in bad[:8]]
    ctx.close()


def test_fp8_append_vs_oracle(orc):
    from oracle import fp8
    p = synth.make_problem(T=333, n_q_heads=24, n_kv_heads=2, seed=41, gate_sigma=2.0)
    got, _, ctx = _fp8_outputs(p, [128, 333])
    want = fp8.attention_fp8(orc, p, threads=8)
    rec = parity_record("fp8 append t333", got, want, p.n_q_heads)
    say(f"  {rec}")
    check_parity(rec)
    ctx.close()


@pytest.mark.parametrize("T,chunks,Hq,Hkv", [(700, [128, 384, 700], 24, 2), (2048, [1024, 1152, 2048], 16, 4)])
def test_fp8_chunks_equal_single_append(T, chunks, Hq, Hkv):
    p = synth.make_problem(T=T, n_q_heads=Hq, n_kv_heads=Hkv, seed=T + 3)
    one, _, c1 = _fp8_outputs(p, [T])
    many, _, c2 = _fp8_outputs(p, chunks)
    assert np.array_equal(one, many)
    c1.close()
    c2.close()


def test_fp8_prefix_workload_sampled(orc):
    """c3's shape over an fp8 cache: keys 0..1023 appended first, then the
    window 1024..8191; sampled window rows against the oracle."""
    from oracle import fp8
    p = cfg("c3_prefix_t8192_qb1024")
    full = synth.make_problem(T=p.T, n_q_heads=p.n_q_heads, n_kv_heads=p.n_kv_heads, seed=p.seed)
    say("fp8 c3 window")
    outs, _, ctx = _fp8_run(full, [p.q_base, p.T])
    got = to_bits(outs[1])
    rows = sample_rows(p.rows, k=16, seed=3)
    want = fp8.attention_fp8(orc, full, rows=rows + p.q_base, threads=8)
    rec = parity_record("fp8 c3 window", got[rows], want, p.n_q_heads, rows)
    say(f"  {rec}")
    check_parity(rec)
    ctx.close()
