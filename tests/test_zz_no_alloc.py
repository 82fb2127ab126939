"""The allocation-free entry point (attn_prefill_gated_noalloc) through the C ABI
against the context entry point (attn_prefill_gated) on the GPU: two calls in a
row, the second smaller than the first (the scratch keeps the first call's
contents), each bit-identical to the context pass, the smaller also within the
contract bound of the oracle; and a call past the scratch limit refused."""

import os
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import DevProblem, check_parity, make_ctx, parity_record, to_bits  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        if os.environ.get("ATTN_REQUIRE_GPU") == "1":
            pytest.fail("ATTN_REQUIRE_GPU=1 but no GPU is visible")
        pytest.skip("no GPU")
    import gated_gqa_causal_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc(ga, p, dp, out):
    geom = ga.geometry(p.n_q_heads, p.n_kv_heads, p.T, p.rms_eps)
    inp = ga.attn_inputs(dp.qg.data_ptr(), dp.k.data_ptr(), dp.v.data_ptr(), dp.wq.data_ptr(), dp.wk.data_ptr(),
                         dp.cos.data_ptr(), dp.sin.data_ptr(), dp.cos.shape[0])
    return ga.attn_prefill_gated_noalloc(geom, inp, p.T, out.data_ptr(), torch.cuda.current_stream().cuda_stream)


def test_noalloc_two_calls_match_the_context_pass(orc):
    import gated_gqa_causal_amd as ga
    big = synth.make_problem(name="noalloc_big", T=8192, n_q_heads=16, n_kv_heads=4, seed=61, gate_sigma=2.0)
    small = synth.make_problem(name="noalloc_small", T=333, n_q_heads=24, n_kv_heads=2, seed=62)
    say("noalloc: 8192 tokens 16/4 (the scratch's full size), then 333 tokens 24/2")
    devs = [DevProblem(big), DevProblem(small)]
    outs = [torch.empty((p.T, p.n_q_heads * 256), dtype=torch.bfloat16, device="cuda") for p in (big, small)]
    for p, dp, out in zip((big, small), devs, outs):
        assert _noalloc(ga, p, dp, out) == ga.ATTN_OK
    torch.cuda.synchronize()
    got = [to_bits(o) for o in outs]
    for p, dp, g in zip((big, small), devs, got):
        ctx = make_ctx(p)
        want = to_bits(ctx.prefill_gated(*dp.args()))
        torch.cuda.synchronize()
        ctx.close()
        same = np.array_equal(g, want)
        say(f"  {p.name}: bit-identical to attn_prefill_gated: {same}")
        assert same
    rec = parity_record("noalloc small vs oracle", got[1], orc.attention(small, threads=8), small.n_q_heads)
    say(f"  {rec}")
    check_parity(rec)


def test_noalloc_refuses_past_the_scratch():
    import gated_gqa_causal_amd as ga
    p = synth.make_problem(name="noalloc_refuse", T=8193, n_q_heads=4, n_kv_heads=4, seed=63)
    dp = DevProblem(p)
    out = torch.empty((p.T, p.n_q_heads * 256), dtype=torch.bfloat16, device="cuda")
    before = out.clone()
    assert _noalloc(ga, p, dp, out) == ga.ATTN_ERR_RANGE
    torch.cuda.synchronize()
    assert torch.equal(out, before)
