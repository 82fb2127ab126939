"""Python binding of libgatedattn.so (MI355X gated GQA causal attention prefill).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/gatedattn.h``.  PyTorch supplies
device memory (``tensor.data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``).  There is no fallback: if the
built library is missing, importing this package raises.

The low-level functions carry the C names (``attn_ctx_create``,
``attn_prefill_gated``, ...).  ``Context`` wraps a context handle and adds
tensor-level calls that check dtype, shape, contiguity and device first.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(_HERE, "libgatedattn.so")

ATTN_ABI_VERSION = 2
ATTN_HEAD_DIM = 256
ATTN_ROTARY_DIM = 64
ATTN_MAX_GROUP = 16
ATTN_MAX_TOKENS = 32768
ATTN_QBASE_ALIGN = 128
ATTN_MAX_SEQS = 4096
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20

ATTN_OK = 0
ATTN_ERR_NULL_ARG = -1
ATTN_ERR_GEOMETRY = -2
ATTN_ERR_RANGE = -3
ATTN_ERR_ALIGN = -4
ATTN_ERR_DEVICE = -5
ATTN_ERR_NOMEM = -6
ATTN_ERR_LAUNCH = -7

ATTN_KERNEL_KV_PROLOGUE = 0
ATTN_KERNEL_MASK_PACK = 1
ATTN_KERNEL_ATTENTION = 2
ATTN_KERNEL_WEIGHTS = 3
ATTN_TIMING_ALL = 15

KIND_GATED, KIND_PREFIX, KIND_MASKED = 0, 1, 2


class attn_geometry(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rotary_dim", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("rms_eps", ctypes.c_float)]


class attn_inputs(ctypes.Structure):
    _fields_ = [("qg", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p),
                ("cos_tab", ctypes.c_void_p), ("sin_tab", ctypes.c_void_p),
                ("n_pos", ctypes.c_int32)]


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {attn_status_string(status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(LIBPATH):
        raise ImportError(f"{LIBPATH} is not built; run __graft_entry__.build() "
                          "(the HIP library is required, there is no fallback)")
    # torch first: its HIP runtime (loaded under the unversioned file name)
    # then satisfies the library's libamdhip64.so.7 dependency by soname.
    # Loaded the other way round, the process would hold two HIP runtimes, and
    # the library's device calls would go to one that does not own torch's
    # device memory and streams (ctx creation then fails on a GPU).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIBPATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    sig = {
        "attn_abi_version": (ctypes.c_int, []),
        "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "attn_validate": (ctypes.c_int, [ctypes.POINTER(attn_geometry), ctypes.POINTER(attn_inputs),
                                         i32, i32, i32, vp, vp]),
        "attn_ctx_create": (ctypes.c_int, [ctypes.POINTER(attn_geometry), ctypes.c_int,
                                           ctypes.POINTER(vp)]),
        "attn_ctx_destroy": (None, [vp]),
        "attn_prefill_gated": (ctypes.c_int, [vp, ctypes.POINTER(attn_inputs), i32, vp, vp]),
        "attn_prefill_gated_noalloc": (ctypes.c_int, [ctypes.POINTER(attn_geometry), ctypes.POINTER(attn_inputs),
                                                      i32, vp, vp]),
        "attn_prefill_prefix": (ctypes.c_int, [vp, ctypes.POINTER(attn_inputs), i32, i32, vp, vp]),
        "attn_prefill_masked": (ctypes.c_int, [vp, ctypes.POINTER(attn_inputs), i32, vp, vp, vp]),
        "attn_prefill_bidirectional": (ctypes.c_int, [vp, ctypes.POINTER(attn_inputs), i32, vp, vp]),
        "attn_validate_weights": (ctypes.c_int, [ctypes.POINTER(attn_geometry), ctypes.POINTER(attn_inputs),
                                                 i32, i32, i32, vp, vp, vp]),
        "attn_prefill_weights": (ctypes.c_int, [vp, ctypes.POINTER(attn_inputs), i32, i32, i32, vp, vp, vp, vp]),
        "attn_kv_cache_bytes": (ctypes.c_int, [ctypes.POINTER(attn_geometry), ctypes.POINTER(ctypes.c_size_t)]),
        "attn_prefill_append": (ctypes.c_int, [vp, ctypes.POINTER(attn_inputs), i32, i32, vp, vp, vp]),
        "attn_kv_cache_fp8_bytes": (ctypes.c_int, [ctypes.POINTER(attn_geometry),
                                                   ctypes.POINTER(ctypes.c_size_t)]),
        "attn_prefill_append_fp8": (ctypes.c_int, [vp, ctypes.POINTER(attn_inputs), i32, i32, vp, vp, vp]),
        "attn_ctx_set_timing": (ctypes.c_int, [vp, ctypes.c_int]),
        "attn_ctx_set_timing_mask": (ctypes.c_int, [vp, ctypes.c_int]),
        "attn_ctx_read_timing": (ctypes.c_int, [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                                ctypes.POINTER(i32)]),
        "attn_mfma_clock_probe": (ctypes.c_int, [i32, vp, ctypes.POINTER(ctypes.c_double),
                                                 ctypes.POINTER(ctypes.c_double)]),
        "attn_validate_batch": (ctypes.c_int, [ctypes.POINTER(attn_geometry), ctypes.POINTER(attn_inputs), i32,
                                               ctypes.POINTER(i32), vp]),
        "attn_prefill_gated_batch": (ctypes.c_int, [vp, ctypes.POINTER(attn_inputs), i32, ctypes.POINTER(i32),
                                                    vp, vp]),
        "attn_validate_shared_batch": (ctypes.c_int, [ctypes.POINTER(attn_geometry), ctypes.POINTER(attn_inputs),
                                                      i32, vp, i32, ctypes.POINTER(i32), vp]),
        "attn_prefill_shared_batch": (ctypes.c_int, [vp, ctypes.POINTER(attn_inputs), i32, vp, i32,
                                                     ctypes.POINTER(i32), vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.attn_abi_version() != ATTN_ABI_VERSION:
        raise ImportError(f"{LIBPATH}: ABI {lib.attn_abi_version()}, expected {ATTN_ABI_VERSION}")
    return lib


lib = _load()


# ---- the C entry points, same names --------------------------------------

def attn_abi_version() -> int:
    return lib.attn_abi_version()


def attn_status_string(status: int) -> str:
    return lib.attn_status_string(status).decode()


def attn_validate(geom: attn_geometry, inputs: Optional[attn_inputs], T: int, q_base: int, kind: int,
                  mask: Optional[int], out: Optional[int]) -> int:
    return lib.attn_validate(ctypes.byref(geom), None if inputs is None else ctypes.byref(inputs),
                             T, q_base, kind, mask, out)


def attn_ctx_create(geom: attn_geometry, device: int) -> int:
    h = ctypes.c_void_p()
    rc = lib.attn_ctx_create(ctypes.byref(geom), device, ctypes.byref(h))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_ctx_create")
    return h.value


def attn_ctx_destroy(ctx: Optional[int]) -> None:
    lib.attn_ctx_destroy(ctx)


def attn_prefill_gated(ctx, inputs: attn_inputs, S: int, out: int, stream: int) -> int:
    return lib.attn_prefill_gated(ctx, ctypes.byref(inputs), S, out, stream)


def attn_prefill_gated_noalloc(geom: attn_geometry, inputs: Optional[attn_inputs], S: int, out: Optional[int],
                               stream: Optional[int]) -> int:
    return lib.attn_prefill_gated_noalloc(ctypes.byref(geom), None if inputs is None else ctypes.byref(inputs),
                                          S, out, stream)


def attn_prefill_prefix(ctx, inputs: attn_inputs, T: int, q_base: int, out: int, stream: int) -> int:
    return lib.attn_prefill_prefix(ctx, ctypes.byref(inputs), T, q_base, out, stream)


def attn_prefill_masked(ctx, inputs: attn_inputs, S: int, mask: int, out: int, stream: int) -> int:
    return lib.attn_prefill_masked(ctx, ctypes.byref(inputs), S, mask, out, stream)


def attn_prefill_bidirectional(ctx, inputs: attn_inputs, S: int, out: int, stream: int) -> int:
    return lib.attn_prefill_bidirectional(ctx, ctypes.byref(inputs), S, out, stream)


def attn_validate_weights(geom: attn_geometry, inputs: Optional[attn_inputs], T: int, q_base: int, kind: int,
                          mask: Optional[int], out: Optional[int], weights: Optional[int]) -> int:
    return lib.attn_validate_weights(ctypes.byref(geom), None if inputs is None else ctypes.byref(inputs),
                                     T, q_base, kind, mask, out, weights)


def attn_prefill_weights(ctx, inputs: attn_inputs, T: int, q_base: int, kind: int, mask: Optional[int], out: int,
                         weights: int, stream: int) -> int:
    return lib.attn_prefill_weights(ctx, ctypes.byref(inputs), T, q_base, kind, mask, out, weights, stream)


def attn_kv_cache_bytes(geom: attn_geometry):
    """(status, bytes) of a K/V cache for the geometry."""
    n = ctypes.c_size_t()
    rc = lib.attn_kv_cache_bytes(ctypes.byref(geom), ctypes.byref(n))
    return rc, n.value


def attn_prefill_append(ctx, inputs: attn_inputs, T: int, q_base: int, kv_cache: int, out: int,
                        stream: int) -> int:
    return lib.attn_prefill_append(ctx, ctypes.byref(inputs), T, q_base, kv_cache, out, stream)


def attn_kv_cache_fp8_bytes(geom: attn_geometry):
    """(status, bytes) of an fp8 K/V cache for the geometry."""
    n = ctypes.c_size_t()
    rc = lib.attn_kv_cache_fp8_bytes(ctypes.byref(geom), ctypes.byref(n))
    return rc, n.value


def attn_prefill_append_fp8(ctx, inputs: attn_inputs, T: int, q_base: int, kv_cache8: int, out: int,
                            stream: int) -> int:
    return lib.attn_prefill_append_fp8(ctx, ctypes.byref(inputs), T, q_base, kv_cache8, out, stream)


def attn_ctx_set_timing(ctx, enable: bool) -> int:
    return lib.attn_ctx_set_timing(ctx, 1 if enable else 0)


def attn_ctx_set_timing_mask(ctx, kernel_mask: int) -> int:
    return lib.attn_ctx_set_timing_mask(ctx, kernel_mask)


def attn_ctx_read_timing(ctx, kernel: int):
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    rc = lib.attn_ctx_read_timing(ctx, kernel, ctypes.byref(ms), ctypes.byref(n))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_ctx_read_timing")
    return ms.value, n.value


def _lens_array(seq_lens):
    n = len(seq_lens)
    return n, (ctypes.c_int32 * max(n, 1))(*[int(x) for x in seq_lens])


def attn_validate_batch(geom: attn_geometry, inputs, seq_lens, out) -> int:
    n, arr = _lens_array(seq_lens)
    return lib.attn_validate_batch(ctypes.byref(geom), ctypes.byref(inputs) if inputs is not None else None, n,
                                   arr, out)


def attn_prefill_gated_batch(ctx, inputs: attn_inputs, seq_lens, out: int, stream: int) -> int:
    n, arr = _lens_array(seq_lens)
    return lib.attn_prefill_gated_batch(ctx, ctypes.byref(inputs), n, arr, out, stream)


def attn_validate_shared_batch(geom: attn_geometry, inputs, prefix_len: int, kv_cache, branch_lens, out) -> int:
    n, arr = _lens_array(branch_lens)
    return lib.attn_validate_shared_batch(ctypes.byref(geom), ctypes.byref(inputs) if inputs is not None else None,
                                          prefix_len, kv_cache, n, arr, out)


def attn_prefill_shared_batch(ctx, inputs: attn_inputs, prefix_len: int, kv_cache, branch_lens, out: int,
                              stream: int) -> int:
    n, arr = _lens_array(branch_lens)
    return lib.attn_prefill_shared_batch(ctx, ctypes.byref(inputs), prefix_len, kv_cache, n, arr, out, stream)


def attn_mfma_clock_probe(iters: int, stream: int = 0):
    """(shader clock MHz, bf16 MFMA TFLOP/s) of the current device under a
    pure matrix-core load with pseudo-random operands (blocking)."""
    mhz = ctypes.c_double()
    tf = ctypes.c_double()
    rc = lib.attn_mfma_clock_probe(iters, stream, ctypes.byref(mhz), ctypes.byref(tf))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_mfma_clock_probe")
    return mhz.value, tf.value


# ---- tensor-level wrapper --------------------------------------------------

def geometry(n_q_heads: int, n_kv_heads: int, max_tokens: int, rms_eps: float = 1e-6) -> attn_geometry:
    return attn_geometry(n_q_heads, n_kv_heads, ATTN_HEAD_DIM, ATTN_ROTARY_DIM, max_tokens, rms_eps)


class Context:
    """One library context bound to a CUDA (HIP) device; owns its workspace."""

    def __init__(self, n_q_heads: int, n_kv_heads: int, max_tokens: int, rms_eps: float = 1e-6,
                 device: Optional[int] = None):
        import torch
        if device is None:
            device = torch.cuda.current_device()
        self.device = int(device)
        self.geom = geometry(n_q_heads, n_kv_heads, max_tokens, rms_eps)
        with torch.cuda.device(self.device):
            self.handle = attn_ctx_create(self.geom, self.device)

    def close(self):
        if getattr(self, "handle", None):
            attn_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- helpers
    def _check(self, name, t, dtype, shape):
        import torch
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.numel() and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() and (t.device.type != "cuda" or t.device.index != self.device):
            raise ValueError(f"{name} must be on cuda:{self.device}")

    def inputs(self, qg, k, v, q_norm_w, k_norm_w, cos, sin, rows: int, T: int) -> attn_inputs:
        import torch
        g = self.geom
        Hq, Hkv, D = g.n_q_heads, g.n_kv_heads, ATTN_HEAD_DIM
        self._check("qg", qg, torch.bfloat16, (rows, Hq, 2, D))
        self._check("k", k, torch.bfloat16, (T, Hkv, D))
        self._check("v", v, torch.bfloat16, (T, Hkv, D))
        self._check("q_norm_w", q_norm_w, torch.bfloat16, (D,))
        self._check("k_norm_w", k_norm_w, torch.bfloat16, (D,))
        if cos.dim() != 2 or cos.shape[1] != ATTN_ROTARY_DIM // 2:
            raise ValueError("cos must be [n_pos][rotary_dim/2]")
        self._check("cos", cos, torch.float32, tuple(cos.shape))
        self._check("sin", sin, torch.float32, tuple(cos.shape))
        return attn_inputs(qg.data_ptr(), k.data_ptr(), v.data_ptr(), q_norm_w.data_ptr(),
                           k_norm_w.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0])

    @staticmethod
    def _stream(stream):
        import torch
        if stream is None:
            return torch.cuda.current_stream().cuda_stream
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)

    def _out(self, out, rows):
        import torch
        g = self.geom
        if out is None:
            out = torch.empty((rows, g.n_q_heads * ATTN_HEAD_DIM), dtype=torch.bfloat16,
                              device=f"cuda:{self.device}")
        self._check("out", out, torch.bfloat16, (rows, g.n_q_heads * ATTN_HEAD_DIM))
        return out

    def prefill_gated(self, qg, k, v, q_norm_w, k_norm_w, cos, sin, out=None, stream=None):
        S = k.shape[0]
        inp = self.inputs(qg, k, v, q_norm_w, k_norm_w, cos, sin, S, S)
        out = self._out(out, S)
        rc = attn_prefill_gated(self.handle, inp, S, out.data_ptr(), self._stream(stream))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_prefill_gated")
        return out

    def prefill_gated_batch(self, qg, k, v, q_norm_w, k_norm_w, cos, sin, seq_lens, out=None, stream=None):
        """Packed batch: the sequences' rows back to back in qg / k / v / out, each
        a causal pass at positions 0..len-1 (seq_lens: host list of lengths)."""
        total = int(sum(int(x) for x in seq_lens))
        inp = self.inputs(qg, k, v, q_norm_w, k_norm_w, cos, sin, total, total)
        out = self._out(out, total)
        rc = attn_prefill_gated_batch(self.handle, inp, list(seq_lens), out.data_ptr(), self._stream(stream))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_prefill_gated_batch")
        return out

    def prefill_shared_batch(self, qg, k, v, q_norm_w, k_norm_w, cos, sin, prefix_len: int, kv_cache, branch_lens,
                             out=None, stream=None):
        """Branches of one shared prefix in one launch: the branches' new rows back to
        back in qg / k / v / out, each at positions prefix_len..prefix_len+len-1 over
        the prefix keys in kv_cache (filled by prefill_append, only read here) and its
        own keys (branch_lens: host list of lengths)."""
        import torch
        total = int(sum(int(x) for x in branch_lens))
        inp = self.inputs(qg, k, v, q_norm_w, k_norm_w, cos, sin, total, total)
        cache_ptr = None
        if kv_cache is not None:
            rc, n = attn_kv_cache_bytes(self.geom)
            if rc != ATTN_OK:
                raise AttnError(rc, "attn_kv_cache_bytes")
            self._check("kv_cache", kv_cache, torch.uint8, (n,))
            cache_ptr = kv_cache.data_ptr()
        out = self._out(out, total)
        rc = attn_prefill_shared_batch(self.handle, inp, prefix_len, cache_ptr, list(branch_lens), out.data_ptr(),
                                       self._stream(stream))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_prefill_shared_batch")
        return out

    def kv_cache(self):
        """A zeroed device K/V cache for this context's geometry (uint8 tensor)."""
        import torch
        rc, n = attn_kv_cache_bytes(self.geom)
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_kv_cache_bytes")
        return torch.zeros(n, dtype=torch.uint8, device=f"cuda:{self.device}")

    def kv_cache_fp8(self):
        """A zeroed device fp8 K/V cache for this context's geometry (uint8 tensor)."""
        import torch
        rc, n = attn_kv_cache_fp8_bytes(self.geom)
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_kv_cache_fp8_bytes")
        return torch.zeros(n, dtype=torch.uint8, device=f"cuda:{self.device}")

    def fp8_cache_views(self, kv_cache8):
        """(key codes [Hkv][tpad][D], value codes, key scales [Hkv][tpad], value scales)
        as views of an fp8 cache tensor."""
        import torch
        g = self.geom
        tpad = (g.max_tokens + 63) // 64 * 64
        rows = g.n_kv_heads * tpad
        D = ATTN_HEAD_DIM
        kc = kv_cache8[:rows * D].view(g.n_kv_heads, tpad, D)
        vc = kv_cache8[rows * D:2 * rows * D].view(g.n_kv_heads, tpad, D)
        sc = kv_cache8[2 * rows * D:].view(torch.float32)
        return kc, vc, sc[:rows].view(g.n_kv_heads, tpad), sc[rows:].view(g.n_kv_heads, tpad)

    def prefill_append_fp8(self, qg, k_new, v_new, q_norm_w, k_norm_w, cos, sin, T: int, q_base: int, kv_cache8,
                           out=None, stream=None):
        """As prefill_append, over an fp8 cache (e4m3 rows with fp32 row scales)."""
        import torch
        rows = T - q_base
        inp = self.inputs(qg, k_new, v_new, q_norm_w, k_norm_w, cos, sin, rows, rows)
        rc, n = attn_kv_cache_fp8_bytes(self.geom)
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_kv_cache_fp8_bytes")
        self._check("kv_cache8", kv_cache8, torch.uint8, (n,))
        out = self._out(out, rows)
        rc = attn_prefill_append_fp8(self.handle, inp, T, q_base, kv_cache8.data_ptr(), out.data_ptr(),
                                     self._stream(stream))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_prefill_append_fp8")
        return out

    def prefill_append(self, qg, k_new, v_new, q_norm_w, k_norm_w, cos, sin, T: int, q_base: int, kv_cache,
                       out=None, stream=None):
        """Rows q_base..T-1 over cache keys 0..T-1; k_new / v_new are the raw rows of
        positions q_base..T-1, prepared into kv_cache by this call."""
        import torch
        rows = T - q_base
        inp = self.inputs(qg, k_new, v_new, q_norm_w, k_norm_w, cos, sin, rows, rows)
        rc, n = attn_kv_cache_bytes(self.geom)
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_kv_cache_bytes")
        self._check("kv_cache", kv_cache, torch.uint8, (n,))
        out = self._out(out, rows)
        rc = attn_prefill_append(self.handle, inp, T, q_base, kv_cache.data_ptr(), out.data_ptr(),
                                 self._stream(stream))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_prefill_append")
        return out

    def prefill_bidirectional(self, qg, k, v, q_norm_w, k_norm_w, cos, sin, out=None, stream=None):
        S = k.shape[0]
        inp = self.inputs(qg, k, v, q_norm_w, k_norm_w, cos, sin, S, S)
        out = self._out(out, S)
        rc = attn_prefill_bidirectional(self.handle, inp, S, out.data_ptr(), self._stream(stream))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_prefill_bidirectional")
        return out

    def prefill_prefix(self, qg, k, v, q_norm_w, k_norm_w, cos, sin, q_base: int, out=None, stream=None):
        T = k.shape[0]
        inp = self.inputs(qg, k, v, q_norm_w, k_norm_w, cos, sin, T - q_base, T)
        out = self._out(out, T - q_base)
        rc = attn_prefill_prefix(self.handle, inp, T, q_base, out.data_ptr(), self._stream(stream))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_prefill_prefix")
        return out

    def prefill_masked(self, qg, k, v, q_norm_w, k_norm_w, cos, sin, mask, out=None, stream=None):
        import torch
        S = k.shape[0]
        inp = self.inputs(qg, k, v, q_norm_w, k_norm_w, cos, sin, S, S)
        self._check("mask", mask, torch.uint8, (S, S))
        out = self._out(out, S)
        rc = attn_prefill_masked(self.handle, inp, S, mask.data_ptr(), out.data_ptr(),
                                 self._stream(stream))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_prefill_masked")
        return out

    def prefill_weights(self, qg, k, v, q_norm_w, k_norm_w, cos, sin, kind: int = 0, q_base: int = 0, mask=None,
                        out=None, weights=None, stream=None):
        """The pass of `kind` (0 gated, 1 prefix window at q_base, 2 masked, 3
        bidirectional) plus its normalised bf16 weights [rows][Hq][T].
        Returns (out, weights)."""
        import torch
        g = self.geom
        T = k.shape[0]
        rows = T - q_base
        inp = self.inputs(qg, k, v, q_norm_w, k_norm_w, cos, sin, rows, T)
        if mask is not None:
            self._check("mask", mask, torch.uint8, (T, T))
        out = self._out(out, rows)
        shape = (rows, g.n_q_heads, T)
        if weights is None:
            weights = torch.empty(shape, dtype=torch.bfloat16, device=f"cuda:{self.device}")
        self._check("weights", weights, torch.bfloat16, shape)
        rc = attn_prefill_weights(self.handle, inp, T, q_base, kind, None if mask is None else mask.data_ptr(),
                                  out.data_ptr(), weights.data_ptr(), self._stream(stream))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_prefill_weights")
        return out, weights

    def set_timing(self, enable: bool, kernels=None):
        """Events around every launch (kernels None) or around the launches of
        the listed ATTN_KERNEL_* ids only; enable False stops."""
        if kernels is None:
            rc = attn_ctx_set_timing(self.handle, enable)
        else:
            rc = attn_ctx_set_timing_mask(self.handle, sum(1 << k for k in set(kernels)) if enable else 0)
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_ctx_set_timing")

    def read_timing(self, kernel: int):
        return attn_ctx_read_timing(self.handle, kernel)
