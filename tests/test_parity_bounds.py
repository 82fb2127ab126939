"""The value-scaled parity bound the GPU tests apply (CPU only).

``gpu_util.check_parity`` asks, besides the contract's 1e-2 + 1e-2|ref| per
element, that the deviation from the oracle stays within 3 quanta rms per
row-head and, per element, within 16 quanta or two bf16 steps of the element,
a quantum being the bf16 spacing at the rms of each row-head's oracle outputs.  These tests show that the bound is both:

* loose enough for a correct kernel: a plain numpy model of the GPU's rounding
  points (the attention-tile page's "Kernel change" recurrence: online softmax
  over 32-key tiles, the unnormalised weight exp2(y - m) rounded to bf16, the
  division by the fp32 row sum at the end; the reference max moved only past a
  threshold of 8 in log2 units) stays within it on rows of the 8192-token
  workload, against the oracle's normalised-weight rounding (the QSA kernel
  page, "Semantics" and final commit message);
* tight enough to fail what the contract bound lets through at long sequences:
  late rows 6% off (one 32-key tile dropped), and the model with a tile dropped.
"""

import numpy as np
import pytest
import torch

import synth
from f64_ref import bf
from gpu_util import check_parity, parity_record, parity_report, row_scale_quanta

ROWS = np.array([3, 40, 1000, 4096, 8191], dtype=np.int32)
LOG2E = np.float32(1.4426950408889634)
SCALE_LOG2 = np.float32(LOG2E * np.float32(0.0625))


def _rb(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


@pytest.fixture(scope="module")
def c2(orc):
    p = synth.config_problem("c2_dense_s8192_g4")
    kp = orc.prepare_keys(p)
    want = orc.attention(p, rows=ROWS, kp=kp, threads=len(ROWS))
    return p, kp, want


def _model(p, kp_bits, qp_bits, rows, drop_tile=None):
    """Gated outputs [len(rows)][Hq*D] (bf16 bits) by the online-softmax rounding
    points; drop_tile (a key-tile index) leaves that tile out of the walk."""
    kp = bf(kp_bits).astype(np.float32)
    qp = bf(qp_bits).astype(np.float32)
    v = bf(p.v).astype(np.float32)
    Hq, G = p.n_q_heads, p.n_q_heads // p.n_kv_heads
    out = np.empty((len(rows), Hq, p.head_dim), np.float32)
    for n, i in enumerate(rows):
        pos = p.q_base + int(i)
        keep = np.ones(pos + 1, bool)
        if drop_tile is not None and 32 * drop_tile <= pos:
            keep[32 * drop_tile:32 * drop_tile + 32] = False
        for h in range(Hq):
            c = h // G
            y = _rb(kp[c, :pos + 1] @ qp[n, h]) * SCALE_LOG2
            m = np.float32(-np.inf)
            for t0 in range(0, pos + 1, 32):
                tm = np.max(np.where(keep[t0:t0 + 32], y[t0:t0 + 32], -np.inf))
                if tm > m + 8:
                    m = tm
            pw = np.where(keep, _rb(np.exp2(y - m)), 0.0).astype(np.float32)
            l = pw.sum(dtype=np.float32)
            o = (pw[:, None] * v[:pos + 1, c]).sum(0, dtype=np.float32)
            ctx = _rb(o * np.float32(1.0 / l))
            g = bf(p.qg[i, h, 1]).astype(np.float64)
            out[n, h] = _rb(ctx * _rb(1.0 / (1.0 + np.exp(-g))))
    return synth.f32_to_bf16_bits(out.reshape(len(rows), -1))


def test_rounding_model_passes(orc, c2):
    p, kp, want = c2
    qp = orc.prepare_queries(synth.Problem(**{**p.__dict__}))[ROWS]
    got = _model(p, kp, qp, ROWS)
    rec = parity_record("numpy model of the online rounding vs oracle", got, want, p.n_q_heads, ROWS)
    print(rec)
    check_parity(rec)


def test_model_with_a_dropped_tile_fails(orc, c2):
    p, kp, want = c2
    rows = ROWS[2:]
    qp = orc.prepare_queries(synth.Problem(**{**p.__dict__}))[rows]
    got = _model(p, kp, qp, rows, drop_tile=17)
    bad, _ = parity_report(got, want[2:])
    assert bad < got.size // 10                      # the contract bound lets it through
    with pytest.raises(AssertionError):
        check_parity(parity_record("model with key tile 17 dropped", got, want[2:], p.n_q_heads))


def test_late_rows_six_percent_off_fail(c2):
    p, _, want = c2
    late = want[2:]
    off = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(late) * np.float32(1.06))
    bad, _ = parity_report(off, late)
    assert bad < off.size // 10
    _, rq, _ = row_scale_quanta(off, late, p.n_q_heads)
    assert rq.min() > 3.0
    with pytest.raises(AssertionError):
        check_parity(parity_record("late rows 6% off", off, late, p.n_q_heads))
