"""Helpers shared by the GPU tests: move a synthetic problem to the device and
run it through the library's C ABI (via the thin Python binding)."""

from __future__ import annotations

import json
import os

import numpy as np
import torch

import synth


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(b)


class DevProblem:
    def __init__(self, p: synth.Problem, device="cuda"):
        self.p = p
        self.qg = bf16_tensor(p.qg, device)
        self.k = bf16_tensor(p.k, device)
        self.v = bf16_tensor(p.v, device)
        self.wq = bf16_tensor(p.q_norm_w, device)
        self.wk = bf16_tensor(p.k_norm_w, device)
        self.cos = torch.from_numpy(np.ascontiguousarray(p.cos)).to(device)
        self.sin = torch.from_numpy(np.ascontiguousarray(p.sin)).to(device)
        self.mask = None if p.mask is None else torch.from_numpy(np.ascontiguousarray(p.mask)).to(device)

    def args(self):
        return (self.qg, self.k, self.v, self.wq, self.wk, self.cos, self.sin)


_TEST_LIB = None


def test_lib():
    """The test build of the library (libgatedattn_test.so: the full C ABI plus
    the test hooks), loaded beside the product library; its contexts are its
    own.  Built by build() next to the product library."""
    global _TEST_LIB
    if _TEST_LIB is None:
        import ctypes
        import gated_gqa_causal_amd as ga      # torch first, then the HIP runtime it loaded
        lib = ctypes.CDLL(ga.LIBPATH.replace("libgatedattn.so", "libgatedattn_test.so"))
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.attn_ctx_create.argtypes = [ctypes.POINTER(ga.attn_geometry), ctypes.c_int, ctypes.POINTER(vp)]
        lib.attn_ctx_create.restype = ctypes.c_int
        lib.attn_ctx_destroy.argtypes = [vp]
        lib.attn_ctx_destroy.restype = None
        lib.attn_debug_prepare.argtypes = [vp, ctypes.POINTER(ga.attn_inputs), i32, i32, vp, vp, vp]
        lib.attn_debug_prepare.restype = ctypes.c_int
        lib.attn_debug_fp8_encode.argtypes = [vp, vp, vp, vp, ctypes.c_int64, vp]
        lib.attn_debug_fp8_encode.restype = ctypes.c_int
        _TEST_LIB = lib
    return _TEST_LIB


def debug_prepare(dp: "DevProblem", q_base: int = 0):
    """Prepared queries [rows][Hq][D] and keys [Hkv][T][D] (bf16 tensors) as the
    kernels compute them, through the test build's attn_debug_prepare."""
    import ctypes
    import gated_gqa_causal_amd as ga
    p = dp.p
    lib = test_lib()
    geom = ga.geometry(p.n_q_heads, p.n_kv_heads, max(p.T, 1), p.rms_eps)
    h = ctypes.c_void_p()
    rc = lib.attn_ctx_create(ctypes.byref(geom), torch.cuda.current_device(), ctypes.byref(h))
    assert rc == ga.ATTN_OK, rc
    inp = ga.attn_inputs(dp.qg.data_ptr(), dp.k.data_ptr(), dp.v.data_ptr(), dp.wq.data_ptr(), dp.wk.data_ptr(),
                         dp.cos.data_ptr(), dp.sin.data_ptr(), dp.cos.shape[0])
    qp = torch.empty((p.T - q_base, p.n_q_heads, 256), dtype=torch.bfloat16, device="cuda")
    kp = torch.empty((p.n_kv_heads, p.T, 256), dtype=torch.bfloat16, device="cuda")
    rc = lib.attn_debug_prepare(h, ctypes.byref(inp), p.T, q_base, qp.data_ptr(), kp.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    lib.attn_ctx_destroy(h)
    assert rc == ga.ATTN_OK, rc
    return qp, kp


def debug_fp8_encode(x: np.ndarray, sc: np.ndarray):
    """(quotients, codes) of the fp8 cache writer's arithmetic for finite rows
    on single values (fp32 arrays x and sc of one length), through the test
    build's attn_debug_fp8_encode."""
    import gated_gqa_causal_amd as ga
    lib = test_lib()
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    sd = torch.from_numpy(np.ascontiguousarray(sc, dtype=np.float32)).cuda()
    q = torch.empty_like(xd)
    codes = torch.empty(xd.shape, dtype=torch.uint8, device="cuda")
    rc = lib.attn_debug_fp8_encode(xd.data_ptr(), sd.data_ptr(), q.data_ptr(), codes.data_ptr(), xd.numel(),
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == ga.ATTN_OK, rc
    return q.cpu().numpy(), codes.cpu().numpy()


def make_ctx(p: synth.Problem, max_tokens=None):
    import gated_gqa_causal_amd as ga
    return ga.Context(p.n_q_heads, p.n_kv_heads, max_tokens or max(p.T, 1), p.rms_eps)


def run(ctx, dp: DevProblem, out=None) -> torch.Tensor:
    p = dp.p
    if p.mask is not None:
        return ctx.prefill_masked(*dp.args(), dp.mask, out=out)
    if not p.causal:
        return ctx.prefill_bidirectional(*dp.args(), out=out)
    if p.q_base:
        return ctx.prefill_prefix(*dp.args(), p.q_base, out=out)
    return ctx.prefill_gated(*dp.args(), out=out)


def gpu_out(p: synth.Problem, ctx=None) -> np.ndarray:
    """Gated output bits [rows][Hq*D] computed on the GPU."""
    own = ctx is None
    ctx = ctx or make_ctx(p)
    dp = DevProblem(p)
    out = run(ctx, dp)
    torch.cuda.synchronize()
    res = to_bits(out)
    if own:
        ctx.close()
    return res


TOL_ABS = 1e-2
TOL_REL = 1e-2


def parity_report(got_bits: np.ndarray, ref_bits: np.ndarray):
    """Element-wise |d| <= 1e-2 + 1e-2 |ref| check; returns (n_bad, worst bound fraction)."""
    g = bits_to_f32(got_bits).astype(np.float64)
    r = bits_to_f32(ref_bits).astype(np.float64)
    bound = TOL_ABS + TOL_REL * np.abs(r)
    err = np.abs(g - r)
    bad = ~(err <= bound)          # NaN counts as bad
    return int(bad.sum()), float(np.nanmax(err / bound)) if err.size else 0.0


# --------------------------------------------------------------------------
# Deviation in row-scale bf16 quanta
# --------------------------------------------------------------------------
# The contract bound above has an absolute floor of 1e-2, which at long
# sequences is as large as the outputs themselves (the late rows of an
# 8192-token pass have a median |out| near 0.005), so it cannot see a wrong
# late row.  The scale that can: the bf16 spacing at the root-mean-square of
# the row-head's 256 oracle outputs, q = 2^(floor(log2 rms) - 7).  The GPU
# rounds the unnormalised weight exp2(y - m) and divides by the row sum at the
# end, where the oracle rounds the normalised weight: each weight differs by at
# most two bf16 roundings, errors of random sign over the keys, so the
# context's deviation has an rms of about u sqrt(sum w^2 v^2), under one or two
# quanta of the row's scale (a numpy model of the two rounding schemes gives
# at most 1.06 over rows of the 8192-token workload; the GPU at most 1.43 over
# every workload and edge case).  A 10% error in a row is at least 12.8 quanta
# rms, a 6% one (one 32-key tile dropped from a late row) at least 7.7, so the
# rms bound sits at 3.  A single element may be off by a bf16 step of its own
# value (a score rounding that flips, summed in another order); an element at
# 8-16x the row's rms has a step of 8-16 quanta, so the element bound is
# max(16 quanta, two steps of the element).
QUANTA_RMS_MAX = 3.0       # per row-head rms of the deviation
QUANTA_ELEM_MAX = 16.0     # any single element (or two bf16 steps of it, if larger)


def row_scale_quanta(got_bits: np.ndarray, ref_bits: np.ndarray, n_heads: int):
    """Deviations in quanta of each row-head's scale.

    Returns (per-element quanta [rows][Hq][D], per row-head rms quanta
    [rows][Hq], mask of row-heads whose oracle outputs are all zero)."""
    g = bits_to_f32(got_bits).astype(np.float64).reshape(got_bits.shape[0], n_heads, -1)
    r = bits_to_f32(ref_bits).astype(np.float64).reshape(ref_bits.shape[0], n_heads, -1)
    rms = np.sqrt(np.mean(r * r, axis=-1))
    zero = rms == 0.0
    q = np.where(zero, 1.0, 2.0 ** (np.floor(np.log2(np.where(zero, 1.0, rms))) - 7))
    d = np.abs(g - r) / q[..., None]
    d = np.where(np.isnan(d), np.inf, d)
    return d, np.sqrt(np.mean(d * d, axis=-1)), zero


def quanta_histogram(d: np.ndarray):
    """Counts of element deviations (row-scale quanta) in the bins 0, (0,1], (1,2], (2,4], (4,8], (8,16], >16."""
    edges = [0.0, 1.0, 2.0, 4.0, 8.0, 16.0]
    h = {"0": int((d == 0).sum())}
    lo = 0.0
    for e in edges[1:]:
        h[f"<={e:g}"] = int(((d > lo) & (d <= e)).sum())
        lo = e
    h[">16"] = int((d > 16.0).sum())
    return h


def parity_record(label: str, got_bits: np.ndarray, ref_bits: np.ndarray, n_heads: int, rows=None):
    """Contract bound + row-scale quanta of one comparison; appends the record to
    the file named by ATTN_PARITY_LOG (one JSON object per line) when set, and
    returns it.  The caller asserts on it with check_parity."""
    bad, frac = parity_report(got_bits, ref_bits)
    d, rq, zero = row_scale_quanta(got_bits, ref_bits, n_heads)
    g = got_bits.reshape(got_bits.shape[0], n_heads, -1)
    r = bits_to_f32(ref_bits).astype(np.float64).reshape(d.shape)
    ar = np.abs(r)
    step = np.where(ar > 0, 2.0 ** (np.floor(np.log2(np.where(ar > 0, ar, 1.0))) - 7), 0.0)
    q = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    q = np.where(q > 0, 2.0 ** (np.floor(np.log2(np.where(q > 0, q, 1.0))) - 7), 1.0)
    outliers = int((d[~zero] * q[~zero] > np.maximum(QUANTA_ELEM_MAX * q[~zero], 2.0 * step[~zero])).sum())
    rec = {
        "case": label, "rows": int(got_bits.shape[0]), "elements": int(got_bits.size),
        "bound_violations": bad, "worst_bound_frac": round(frac, 4),
        "rms_quanta_max": round(float(rq[~zero].max()) if (~zero).any() else 0.0, 3),
        "rms_quanta_median": round(float(np.median(rq[~zero])) if (~zero).any() else 0.0, 3),
        "elem_quanta_max": round(float(d[~zero].max()) if (~zero).any() else 0.0, 2),
        "elem_outliers": outliers,
        "hist": quanta_histogram(d[~zero]),
        "zero_rows_nonzero": int((g[zero] != 0).sum()),
        "identical": round(float(np.mean(got_bits == ref_bits)), 4),
    }
    if rows is not None:
        rec["first_rows"] = [int(x) for x in np.asarray(rows)[:4]]
    path = os.environ.get("ATTN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    return rec


def check_parity_either_reading(orc, p, got_bits: np.ndarray, label: str, rows=None, threads: int = 8):
    """check_parity against the oracle, where a row-head over the row-scale bounds
    may instead meet them against the oracle's other reading of the score's dot
    product (summed in double, rounded once to fp32).  The pages fix the score as
    the bf16 rounding of an fp32 dot product, not the order of its sum: a key whose
    exact dot product lies within the fp32 summation error of a bf16 tie can round
    either way, and when it carries much of the row's weight the whole row-head
    moves by several quanta.  The contract bound and exact zeros are checked
    against the default reading.  Returns the default reading's record, with the
    count of row-heads that needed the other one."""
    want = orc.attention(p, rows=rows, threads=threads)
    rec = parity_record(label, got_bits, want, p.n_q_heads, rows)
    assert rec["bound_violations"] == 0, rec
    assert rec["zero_rows_nonzero"] == 0, rec
    d, rq, zero = row_scale_quanta(got_bits, want, p.n_q_heads)
    r = bits_to_f32(want).astype(np.float64).reshape(d.shape)
    ar = np.abs(r)
    step = np.where(ar > 0, 2.0 ** (np.floor(np.log2(np.where(ar > 0, ar, 1.0))) - 7), 0.0)
    q = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    q = np.where(q > 0, 2.0 ** (np.floor(np.log2(np.where(q > 0, q, 1.0))) - 7), 1.0)
    elem_bad = (d * q > np.maximum(QUANTA_ELEM_MAX * q, 2.0 * step)).any(axis=-1)
    bad = ~zero & ((rq > QUANTA_RMS_MAX) | elem_bad)
    rec["other_reading_row_heads"] = int(bad.sum())
    if bad.any():
        bad_rows = np.nonzero(bad.any(axis=1))[0]
        all_rows = np.arange(got_bits.shape[0]) if rows is None else np.asarray(rows)
        alt = orc.attention(p, rows=np.asarray(all_rows)[bad_rows].astype(np.int32), threads=threads,
                            score_f64=True)
        sub = parity_record(label + " (other reading, flagged rows)", got_bits[bad_rows], alt, p.n_q_heads)
        d2, rq2, zero2 = row_scale_quanta(got_bits[bad_rows], alt, p.n_q_heads)
        r2 = bits_to_f32(alt).astype(np.float64).reshape(d2.shape)
        ar2 = np.abs(r2)
        step2 = np.where(ar2 > 0, 2.0 ** (np.floor(np.log2(np.where(ar2 > 0, ar2, 1.0))) - 7), 0.0)
        q2 = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True))
        q2 = np.where(q2 > 0, 2.0 ** (np.floor(np.log2(np.where(q2 > 0, q2, 1.0))) - 7), 1.0)
        elem_bad2 = (d2 * q2 > np.maximum(QUANTA_ELEM_MAX * q2, 2.0 * step2)).any(axis=-1)
        still = bad[bad_rows] & ((rq2 > QUANTA_RMS_MAX) | elem_bad2)
        assert not still.any(), (rec, sub)
        rec["other_reading_rms_quanta_max"] = round(float(rq2[bad[bad_rows]].max()), 3)
    return rec


def check_parity(rec):
    """The contract bound on every element, the row-scale quanta bounds (rms per
    row-head, and each element within max(16 quanta, two bf16 steps of itself)),
    and exact zeros where the oracle's row-head is all zero (no visible key)."""
    assert rec["bound_violations"] == 0, rec
    assert rec["zero_rows_nonzero"] == 0, rec
    assert rec["rms_quanta_max"] <= QUANTA_RMS_MAX, rec
    assert rec["elem_outliers"] == 0, rec
