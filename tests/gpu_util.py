"""Helpers shared by the GPU tests: move a synthetic problem to the device and
run it through the library's C ABI (via the thin Python binding)."""

from __future__ import annotations

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
