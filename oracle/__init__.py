"""CPU oracle for gated GQA causal attention prefill (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  It wraps ``oracle.c`` (plain C, fp32 with the bf16 rounding
points of the reference model, every sum in ascending order) through ctypes
and shares nothing with the HIP library except the seeded inputs from
``synth``.

``oracle/fp8.py`` adds the fp8 (E4M3) K/V cache rows (per-row fp32 scale,
widened to bf16) as plain numpy; its pins are in ``tests/test_fp8_pins.py``.

Parity pins live in ``tests/test_oracle_pins.py``.  One part is unpinned
(parity unpinned): absolute fidelity to the pages' own reference model, whose
golden fixture is not available; the rotate-half pairing and the bf16 rounding
of the RoPE products rest on the pages' prose alone.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBPATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing", "-std=c11",
          "-shared", "-fPIC"]


def build(out: str = LIBPATH, mutation: int = 0) -> str:
    """Compiles oracle.c with gcc (optionally with one planted mutation)."""
    cmd = ["gcc", *CFLAGS, f"-DORACLE_MUTATION={int(mutation)}", SOURCE, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("rotary_dim", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("T", ctypes.c_int32), ("q_base", ctypes.c_int32),
        ("qg", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p),
        ("cos_tab", ctypes.c_void_p), ("sin_tab", ctypes.c_void_p),
        ("n_pos", ctypes.c_int32),
        ("mask", ctypes.c_void_p), ("kp", ctypes.c_void_p),
        ("causal", ctypes.c_int32),
        ("score_f64", ctypes.c_int32),
    ]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


ORACLE_ABI = 3      # layout of _Problem; oracle.c's oracle_abi() must agree


class Oracle:
    """Handle on one build of the oracle library.  The default library is
    (re)built when it is missing or older than oracle.c."""

    def __init__(self, libpath: str = LIBPATH):
        if libpath == LIBPATH:
            if not os.path.exists(libpath) or os.path.getmtime(libpath) < os.path.getmtime(SOURCE):
                build()
        elif not os.path.exists(libpath):
            raise FileNotFoundError(libpath)
        self.lib = ctypes.CDLL(libpath)
        L = self.lib
        if L.oracle_abi() != ORACLE_ABI:
            raise RuntimeError(f"{libpath}: oracle ABI {L.oracle_abi()}, expected {ORACLE_ABI}; rebuild it")
        L.oracle_bf16_round.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.oracle_norm_rope.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int32, ctypes.c_int32,
                                                               ctypes.c_float, ctypes.c_void_p]
        L.oracle_prepare_keys.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p]
        L.oracle_prepare_queries.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p]
        L.oracle_attention.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
        self.mutation = L.oracle_mutation()

    # ---- primitives -------------------------------------------------------
    def bf16_round(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_bf16_round(_ptr(x), _ptr(out), x.size)
        return out

    def norm_rope(self, x, w, cos_row, sin_row, rotary_dim: int = 64, eps: float = 1e-6):
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        c = np.ascontiguousarray(cos_row, dtype=np.float32)
        s = np.ascontiguousarray(sin_row, dtype=np.float32)
        out = np.empty(x.shape[-1], dtype=np.uint16)
        self.lib.oracle_norm_rope(_ptr(x), _ptr(w), _ptr(c), _ptr(s), x.shape[-1], rotary_dim,
                                  eps, _ptr(out))
        return out

    # ---- whole problems ---------------------------------------------------
    def _struct(self, p, kp=None, keep=None):
        arrs = dict(qg=np.ascontiguousarray(p.qg, dtype=np.uint16),
                    k=np.ascontiguousarray(p.k, dtype=np.uint16),
                    v=np.ascontiguousarray(p.v, dtype=np.uint16),
                    wq=np.ascontiguousarray(p.q_norm_w, dtype=np.uint16),
                    wk=np.ascontiguousarray(p.k_norm_w, dtype=np.uint16),
                    cos=np.ascontiguousarray(p.cos, dtype=np.float32),
                    sin=np.ascontiguousarray(p.sin, dtype=np.float32),
                    mask=None if p.mask is None else np.ascontiguousarray(p.mask, dtype=np.uint8),
                    kp=kp)
        if keep is not None:
            keep.update(arrs)
        s = _Problem(p.n_q_heads, p.n_kv_heads, p.head_dim, p.rotary_dim, p.rms_eps, p.T,
                     p.q_base, _ptr(arrs["qg"]), _ptr(arrs["k"]), _ptr(arrs["v"]),
                     _ptr(arrs["wq"]), _ptr(arrs["wk"]), _ptr(arrs["cos"]), _ptr(arrs["sin"]),
                     arrs["cos"].shape[0], _ptr(arrs["mask"]), _ptr(kp),
                     1 if getattr(p, "causal", True) else 0, 0)
        return s, arrs

    def prepare_keys(self, p) -> np.ndarray:
        """Prepared keys [Hkv][T][D] (bf16 bits)."""
        kp = np.empty((p.n_kv_heads, p.T, p.head_dim), dtype=np.uint16)
        s, _keep = self._struct(p)
        if self.lib.oracle_prepare_keys(ctypes.byref(s), _ptr(kp)) != 0:
            raise ValueError("oracle_prepare_keys refused the problem")
        return kp

    def prepare_queries(self, p) -> np.ndarray:
        """Prepared queries [rows][Hq][D] (bf16 bits)."""
        qp = np.empty((p.rows, p.n_q_heads, p.head_dim), dtype=np.uint16)
        s, _keep = self._struct(p)
        if self.lib.oracle_prepare_queries(ctypes.byref(s), _ptr(qp)) != 0:
            raise ValueError("oracle_prepare_queries refused the problem")
        return qp

    def attention(self, p, rows: Optional[Sequence[int]] = None, *, kp: Optional[np.ndarray] = None,
                  want_ctx: bool = False, want_wsum: bool = False, want_weights: bool = False,
                  threads: int = 1, score_f64: bool = False):
        """Gated outputs [n_rows][Hq*D] (bf16 bits) for the listed window rows.

        ``score_f64`` takes the other reading of the score's dot product (summed
        in double and rounded once to fp32, instead of ascending fp32 sums); the
        rest of the arithmetic is unchanged.

        Returns ``out`` alone, or a dict with ``out`` plus the requested
        intermediates (``ctx``, ``wsum``, ``weights``).  ``threads`` spreads
        independent rows over host threads; each (row, head) unit is computed
        exactly as on one thread.
        """
        if kp is None:
            kp = self.prepare_keys(p)
        rows = np.arange(p.rows, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
        n, Hq, D, T = rows.size, p.n_q_heads, p.head_dim, p.T
        out = np.empty((n, Hq * D), dtype=np.uint16)
        ctx = np.empty((n, Hq * D), dtype=np.uint16) if want_ctx else None
        wsum = np.empty((n, Hq), dtype=np.float32) if want_wsum else None
        wts = np.empty((n, Hq, T), dtype=np.float32) if want_weights else None
        s, keep = self._struct(p, kp=np.ascontiguousarray(kp, dtype=np.uint16))
        s.score_f64 = 1 if score_f64 else 0
        errors = []

        def run(a: int, b: int):
            if b <= a:
                return
            rr = np.ascontiguousarray(rows[a:b])
            sub = lambda x: None if x is None else x[a:b].ctypes.data_as(ctypes.c_void_p)
            rc = self.lib.oracle_attention(ctypes.byref(s), _ptr(rr), b - a, sub(out), sub(ctx),
                                           sub(wsum), sub(wts))
            if rc != 0:
                errors.append(rc)

        threads = max(1, min(int(threads), n if n else 1))
        if threads == 1:
            run(0, n)
        else:
            # Interleave rows so the triangular work spreads evenly.
            order = np.argsort(-rows.astype(np.int64), kind="stable")
            buckets = [order[t::threads] for t in range(threads)]
            results = []
            lock = threading.Lock()

            def run_bucket(idx):
                sub_rows = rows[idx]
                o = np.empty((idx.size, Hq * D), dtype=np.uint16)
                c = np.empty((idx.size, Hq * D), dtype=np.uint16) if want_ctx else None
                w = np.empty((idx.size, Hq), dtype=np.float32) if want_wsum else None
                wt = np.empty((idx.size, Hq, T), dtype=np.float32) if want_weights else None
                rc = self.lib.oracle_attention(ctypes.byref(s), _ptr(np.ascontiguousarray(sub_rows)),
                                               idx.size, _ptr(o), _ptr(c), _ptr(w), _ptr(wt))
                with lock:
                    results.append((idx, o, c, w, wt, rc))

            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run_bucket, buckets))
            for idx, o, c, w, wt, rc in results:
                if rc != 0:
                    errors.append(rc)
                out[idx] = o
                if want_ctx:
                    ctx[idx] = c
                if want_wsum:
                    wsum[idx] = w
                if want_weights:
                    wts[idx] = wt
        del keep
        if errors:
            raise ValueError(f"oracle_attention refused the problem ({errors[0]})")
        if not (want_ctx or want_wsum or want_weights):
            return out
        res = {"out": out}
        if want_ctx:
            res["ctx"] = ctx
        if want_wsum:
            res["wsum"] = wsum
        if want_weights:
            res["weights"] = wts
        return res


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
