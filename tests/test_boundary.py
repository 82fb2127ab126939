"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
refuses bad calls with the documented status before touching any device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gatedattn.h")


@pytest.fixture(scope="module")
def ga():
    import gated_gqa_causal_amd
    return gated_gqa_causal_amd


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"ATTN_EXPORT\s+[\w\s\*]*?\b(attn_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["attn_ctx_create", "attn_prefill_gated", "attn_prefill_prefix", "attn_prefill_masked",
              "attn_prefill_bidirectional", "attn_prefill_append", "attn_kv_cache_bytes", "attn_ctx_destroy",
              "attn_abi_version", "attn_status_string", "attn_validate"]:
        assert n in names


def test_library_exports_every_declared_symbol(ga):
    lib = ctypes.CDLL(ga.LIBPATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


def test_header_constants_match_binding(ga):
    src = open(HEADER).read()
    for name in ["ATTN_ABI_VERSION", "ATTN_HEAD_DIM", "ATTN_ROTARY_DIM", "ATTN_MAX_GROUP",
                 "ATTN_MAX_TOKENS", "ATTN_QBASE_ALIGN", "ATTN_MAX_SEQS", "ATTN_KERNEL_KV_PROLOGUE",
                 "ATTN_KERNEL_MASK_PACK", "ATTN_KERNEL_ATTENTION", "ATTN_KERNEL_WEIGHTS", "ATTN_TIMING_ALL"]:
        m = re.search(rf"#define {name}\s+(\d+)", src)
        assert m and int(m.group(1)) == getattr(ga, name), name
    for name in ["ATTN_OK", "ATTN_ERR_NULL_ARG", "ATTN_ERR_GEOMETRY", "ATTN_ERR_RANGE",
                 "ATTN_ERR_ALIGN", "ATTN_ERR_DEVICE", "ATTN_ERR_NOMEM", "ATTN_ERR_LAUNCH"]:
        m = re.search(rf"{name}\s*=\s*(-?\d+)", src)
        assert m and int(m.group(1)) == getattr(ga, name), name
    assert ga.attn_abi_version() == ga.ATTN_ABI_VERSION


def test_status_strings(ga):
    for s in range(-7, 1):
        assert ga.attn_status_string(s) not in ("", "unknown status")
    assert ga.attn_status_string(-99) == "unknown status"


FAKE = 0x1000   # 16-byte aligned, never dereferenced: validation is host-only


def _inputs(ga, n_pos=64, base=FAKE):
    return ga.attn_inputs(base, base, base, base, base, base, base, n_pos)


def _geom(ga, **kw):
    g = dict(n_q_heads=24, n_kv_heads=2, max_tokens=256, rms_eps=1e-6)
    g.update(kw)
    return ga.geometry(**g)


REFUSALS = [
    # (geometry overrides, T, q_base, kind, mask, out, inputs overrides, expected)
    (dict(n_q_heads=24, n_kv_heads=5), 64, 0, 0, None, FAKE, {}, "GEOMETRY"),
    (dict(n_q_heads=34, n_kv_heads=2), 64, 0, 0, None, FAKE, {}, "GEOMETRY"),   # G = 17
    (dict(rms_eps=0.0), 64, 0, 0, None, FAKE, {}, "GEOMETRY"),
    (dict(rms_eps=float("nan")), 64, 0, 0, None, FAKE, {}, "GEOMETRY"),
    (dict(max_tokens=0), 0, 0, 0, None, FAKE, {}, "RANGE"),
    (dict(max_tokens=40000), 64, 0, 0, None, FAKE, {}, "RANGE"),
    ({}, 257, 0, 0, None, FAKE, {}, "RANGE"),                      # T > max_tokens
    ({}, -1, 0, 0, None, FAKE, {}, "RANGE"),
    ({}, 200, 256, 1, None, FAKE, {}, "RANGE"),                    # q_base > T
    ({}, 200, 64, 1, None, FAKE, {}, "ALIGN"),                     # q_base % 128
    ({}, 200, 128, 0, None, FAKE, {}, "RANGE"),                    # q_base on the full pass
    ({}, 200, 0, 6, None, FAKE, {}, "RANGE"),                      # bad kind
    ({}, 200, 128, 5, None, FAKE, dict(n_pos=256), "NULL_ARG"),    # fp8 append without a cache
    ({}, 200, 128, 5, FAKE + 4, FAKE, dict(n_pos=256), "ALIGN"),   # misaligned fp8 cache
    ({}, 200, 64, 5, FAKE, FAKE, dict(n_pos=256), "ALIGN"),        # fp8 append q_base % 128
    ({}, 200, 0, -1, None, FAKE, {}, "RANGE"),                     # negative kind
    ({}, 200, -128, 1, None, FAKE, {}, "RANGE"),                   # negative q_base
    ({}, 200, 128, 3, None, FAKE, {}, "RANGE"),                    # q_base on the bidirectional pass
    ({}, 64, 0, 3, None, FAKE, dict(v=0), "NULL_ARG"),
    ({}, 200, 128, 4, None, FAKE, dict(n_pos=256), "NULL_ARG"),    # append without a cache
    ({}, 200, 128, 4, FAKE + 4, FAKE, dict(n_pos=256), "ALIGN"),   # misaligned cache
    ({}, 200, 64, 4, FAKE, FAKE, dict(n_pos=256), "ALIGN"),        # append q_base % 128
    ({}, 200, 256, 4, FAKE, FAKE, dict(n_pos=256), "RANGE"),       # append q_base > T
    ({}, 64, 0, 0, None, FAKE, dict(n_pos=63), "RANGE"),           # short cos/sin table
    ({}, 64, 0, 0, None, None, {}, "NULL_ARG"),                    # out
    ({}, 64, 0, 2, None, FAKE, {}, "NULL_ARG"),                    # mask
    ({}, 64, 0, 0, None, FAKE, dict(qg=0), "NULL_ARG"),
    ({}, 64, 0, 0, None, FAKE, dict(k=0), "NULL_ARG"),
    ({}, 64, 0, 0, None, FAKE, dict(v=0), "NULL_ARG"),
    ({}, 64, 0, 0, None, FAKE, dict(q_norm_w=0), "NULL_ARG"),
    ({}, 64, 0, 0, None, FAKE, dict(k_norm_w=0), "NULL_ARG"),
    ({}, 64, 0, 0, None, FAKE, dict(cos_tab=0), "NULL_ARG"),
    ({}, 64, 0, 0, None, FAKE, dict(sin_tab=0), "NULL_ARG"),
    ({}, 64, 0, 0, None, FAKE + 8, {}, "ALIGN"),                   # out misaligned
    ({}, 64, 0, 0, None, FAKE, dict(qg=FAKE + 2), "ALIGN"),
]


@pytest.mark.parametrize("case", REFUSALS, ids=lambda c: f"{c[-1]}")
def test_refusals(ga, case):
    geo, T, qb, kind, mask, out, inov, want = case
    inp = _inputs(ga)
    for k, v in inov.items():
        setattr(inp, k, v)
    rc = ga.attn_validate(_geom(ga, **geo), inp, T, qb, kind, mask, out)
    assert rc == getattr(ga, "ATTN_ERR_" + want), (rc, ga.attn_status_string(rc))


def test_null_geometry(ga):
    rc = ga.lib.attn_validate(None, None, 0, 0, 0, None, None)
    assert rc == ga.ATTN_ERR_NULL_ARG


@pytest.mark.parametrize("T,qb,kind", [(0, 0, 0), (0, 0, 2), (256, 256, 1), (128, 128, 1), (0, 0, 3),
                                       (128, 128, 4), (256, 256, 5)])
def test_empty_launch_is_ok_without_pointers(ga, T, qb, kind):
    # Zero query rows: a no-op, even with every pointer NULL (torch gives 0 for empty tensors).
    assert ga.attn_validate(_geom(ga), None, T, qb, kind, None, None) == ga.ATTN_OK


def test_valid_calls_pass(ga):
    assert ga.attn_validate(_geom(ga), _inputs(ga, 256), 256, 0, 0, None, FAKE) == ga.ATTN_OK
    assert ga.attn_validate(_geom(ga), _inputs(ga, 256), 256, 128, 1, None, FAKE) == ga.ATTN_OK
    assert ga.attn_validate(_geom(ga), _inputs(ga, 256), 256, 0, 2, FAKE + 3, FAKE) == ga.ATTN_OK
    assert ga.attn_validate(_geom(ga), _inputs(ga, 256), 256, 0, 3, None, FAKE) == ga.ATTN_OK
    assert ga.attn_validate(_geom(ga), _inputs(ga, 256), 256, 128, 4, FAKE, FAKE) == ga.ATTN_OK
    assert ga.attn_validate(_geom(ga), _inputs(ga, 256), 256, 0, 4, FAKE, FAKE) == ga.ATTN_OK
    assert ga.attn_validate(_geom(ga), _inputs(ga, 256), 256, 128, 5, FAKE, FAKE) == ga.ATTN_OK
    for G in [1, 2, 3, 12, 16]:
        assert ga.attn_validate(_geom(ga, n_q_heads=2 * G), _inputs(ga), 64, 0, 0, None, FAKE) == 0


def test_null_context_refused(ga):
    inp = _inputs(ga)
    assert ga.attn_prefill_gated(None, inp, 64, FAKE, None) == ga.ATTN_ERR_NULL_ARG
    assert ga.attn_prefill_prefix(None, inp, 64, 0, FAKE, None) == ga.ATTN_ERR_NULL_ARG
    assert ga.attn_prefill_masked(None, inp, 64, FAKE, FAKE, None) == ga.ATTN_ERR_NULL_ARG
    assert ga.attn_prefill_bidirectional(None, inp, 64, FAKE, None) == ga.ATTN_ERR_NULL_ARG
    assert ga.attn_prefill_append(None, inp, 256, 128, FAKE, FAKE, None) == ga.ATTN_ERR_NULL_ARG
    assert ga.attn_ctx_set_timing(None, 1) == ga.ATTN_ERR_NULL_ARG
    assert ga.attn_ctx_set_timing_mask(None, 1 << ga.ATTN_KERNEL_ATTENTION) == ga.ATTN_ERR_NULL_ARG
    ga.attn_ctx_destroy(None)      # no-op


def test_create_refuses_bad_geometry_before_device(ga):
    with pytest.raises(ga.AttnError) as e:
        ga.attn_ctx_create(_geom(ga, n_q_heads=5, n_kv_heads=2), 0)
    assert e.value.status == ga.ATTN_ERR_GEOMETRY


def test_create_without_a_device_fails_cleanly(ga):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(ga.AttnError) as e:
        ga.attn_ctx_create(_geom(ga), 0)
    assert e.value.status == ga.ATTN_ERR_DEVICE


def test_kv_cache_bytes(ga):
    g = _geom(ga, n_q_heads=16, n_kv_heads=4, max_tokens=1000)
    rc, n = ga.attn_kv_cache_bytes(g)
    assert rc == ga.ATTN_OK
    assert n == 2 * 4 * 1024 * 256 * 2          # K and V^T, max_tokens rounded up to 64
    rc, n = ga.attn_kv_cache_bytes(_geom(ga, n_q_heads=24, n_kv_heads=5))
    assert rc == ga.ATTN_ERR_GEOMETRY and n == 0
    assert ga.lib.attn_kv_cache_bytes(g, None) == ga.ATTN_ERR_NULL_ARG


def test_mfma_probe_refuses_bad_arguments(ga):
    """The calibration entry checks its arguments before touching a device."""
    mhz, tf = ctypes.c_double(), ctypes.c_double()
    assert ga.lib.attn_mfma_clock_probe(0, None, ctypes.byref(mhz), ctypes.byref(tf)) == ga.ATTN_ERR_RANGE
    assert ga.lib.attn_mfma_clock_probe(10 ** 8, None, ctypes.byref(mhz), ctypes.byref(tf)) == ga.ATTN_ERR_RANGE
    assert ga.lib.attn_mfma_clock_probe(10, None, None, ctypes.byref(tf)) == ga.ATTN_ERR_NULL_ARG


BATCH_REFUSALS = [
    # (geometry overrides, seq_lens, out, inputs overrides, expected)
    ({}, [64, -1], FAKE, {}, "RANGE"),                         # negative length
    ({}, [200, 57], FAKE, {}, "RANGE"),                        # total > max_tokens (256)
    ({}, [257], FAKE, {}, "RANGE"),                            # one length > max_tokens
    (dict(max_tokens=64), [1, 1, 1], FAKE, {}, "RANGE"),       # 3 tiles of 32 > 64 keys of workspace
    ({}, [64, 100], FAKE, dict(n_pos=99), "RANGE"),            # table shorter than the longest sequence
    ({}, [64, 100], None, {}, "NULL_ARG"),
    ({}, [64, 100], FAKE, dict(k=0), "NULL_ARG"),
    ({}, [64, 100], FAKE + 8, {}, "ALIGN"),
    (dict(n_q_heads=24, n_kv_heads=5), [64], FAKE, {}, "GEOMETRY"),
]


@pytest.mark.parametrize("case", BATCH_REFUSALS, ids=lambda c: f"{c[-1]}")
def test_batch_refusals(ga, case):
    geo, lens, out, inov, want = case
    inp = _inputs(ga, n_pos=256)
    for k, v in inov.items():
        setattr(inp, k, v)
    rc = ga.attn_validate_batch(_geom(ga, **geo), inp, lens, out)
    assert rc == getattr(ga, "ATTN_ERR_" + want), (rc, ga.attn_status_string(rc))


def test_batch_count_limits(ga):
    g = _geom(ga)
    n = ctypes.c_int32(1)
    assert ga.lib.attn_validate_batch(ctypes.byref(g), None, -1, None, None) == ga.ATTN_ERR_RANGE
    assert ga.lib.attn_validate_batch(ctypes.byref(g), None, ga.ATTN_MAX_SEQS + 1, None, None) == ga.ATTN_ERR_RANGE
    assert ga.lib.attn_validate_batch(ctypes.byref(g), None, 1, None, None) == ga.ATTN_ERR_NULL_ARG
    assert ga.lib.attn_validate_batch(ctypes.byref(g), None, 1, ctypes.byref(n), None) == ga.ATTN_ERR_NULL_ARG
    # ATTN_MAX_SEQS zero-length sequences: a no-op
    assert ga.attn_validate_batch(g, None, [0] * ga.ATTN_MAX_SEQS, None) == ga.ATTN_OK


def test_batch_valid_and_empty(ga):
    g = _geom(ga)
    assert ga.attn_validate_batch(g, None, [], None) == ga.ATTN_OK
    assert ga.attn_validate_batch(g, None, [0, 0], None) == ga.ATTN_OK
    assert ga.attn_validate_batch(g, _inputs(ga, n_pos=100), [64, 0, 100, 31], FAKE) == ga.ATTN_OK
    # 8 sequences of 32 fill the 256-key workspace exactly
    assert ga.attn_validate_batch(g, _inputs(ga, n_pos=32), [32] * 8, FAKE) == ga.ATTN_OK
    assert ga.attn_validate_batch(g, _inputs(ga, n_pos=33), [32] * 7 + [1, 1], FAKE) == ga.ATTN_ERR_RANGE


SHARED_REFUSALS = [
    # (geometry overrides, prefix_len, cache, branch_lens, out, inputs overrides, expected)
    ({}, 64, FAKE, [10], FAKE, {}, "ALIGN"),                   # prefix not a multiple of ATTN_QBASE_ALIGN
    ({}, -128, FAKE, [10], FAKE, {}, "RANGE"),
    ({}, 384, FAKE, [10], FAKE, {}, "RANGE"),                  # prefix past max_tokens (256)
    ({}, 128, FAKE, [64, 129], FAKE, {}, "RANGE"),             # 128 + 129 positions > max_tokens
    ({}, 128, FAKE, [64, -1], FAKE, {}, "RANGE"),
    ({}, 0, FAKE, [200, 57], FAKE, {}, "RANGE"),               # new tokens > max_tokens
    ({}, 128, FAKE, [64, 100], FAKE, dict(n_pos=227), "RANGE"),  # table shorter than prefix + longest branch
    ({}, 128, None, [64, 100], FAKE, {}, "NULL_ARG"),          # a prefix needs its cache
    ({}, 128, FAKE, [64, 100], None, {}, "NULL_ARG"),
    ({}, 128, FAKE, [64, 100], FAKE, dict(v=0), "NULL_ARG"),
    ({}, 128, FAKE + 8, [64, 100], FAKE, {}, "ALIGN"),
    ({}, 128, FAKE, [64, 100], FAKE + 8, {}, "ALIGN"),
    (dict(n_q_heads=24, n_kv_heads=5), 128, FAKE, [64], FAKE, {}, "GEOMETRY"),
]


@pytest.mark.parametrize("case", SHARED_REFUSALS, ids=lambda c: f"{c[-1]}")
def test_shared_batch_refusals(ga, case):
    geo, P, cache, lens, out, inov, want = case
    inp = _inputs(ga, n_pos=256)
    for k, v in inov.items():
        setattr(inp, k, v)
    rc = ga.attn_validate_shared_batch(_geom(ga, **geo), inp, P, cache, lens, out)
    assert rc == getattr(ga, "ATTN_ERR_" + want), (rc, ga.attn_status_string(rc))


def test_shared_batch_valid_and_empty(ga):
    g = _geom(ga)
    # nothing new: a no-op whatever the pointers (a misaligned prefix still refused first)
    assert ga.attn_validate_shared_batch(g, None, 128, None, [], None) == ga.ATTN_OK
    assert ga.attn_validate_shared_batch(g, None, 128, None, [0, 0], None) == ga.ATTN_OK
    assert ga.attn_validate_shared_batch(g, None, 64, None, [0], None) == ga.ATTN_ERR_ALIGN
    assert ga.attn_validate_shared_batch(g, _inputs(ga, n_pos=228), 128, FAKE, [64, 0, 100, 31], FAKE) == ga.ATTN_OK
    # the branches' own keys fill the 256-key workspace exactly
    assert ga.attn_validate_shared_batch(g, _inputs(ga, n_pos=160), 128, FAKE, [32] * 8, FAKE) == ga.ATTN_OK
    assert ga.attn_validate_shared_batch(g, _inputs(ga, n_pos=160), 128, FAKE, [32] * 7 + [1, 1], FAKE) == \
        ga.ATTN_ERR_RANGE
    # no prefix: a plain packed batch, the cache unused
    assert ga.attn_validate_shared_batch(g, _inputs(ga, n_pos=100), 0, None, [64, 100], FAKE) == ga.ATTN_OK
    n = ctypes.c_int32(1)
    assert ga.lib.attn_validate_shared_batch(ctypes.byref(g), None, 128, None, ga.ATTN_MAX_SEQS + 1, None,
                                             None) == ga.ATTN_ERR_RANGE
    assert ga.lib.attn_validate_shared_batch(ctypes.byref(g), None, 128, None, 1, None, None) == \
        ga.ATTN_ERR_NULL_ARG
    assert ga.lib.attn_validate_shared_batch(ctypes.byref(g), None, 128, None, 1, ctypes.byref(n), None) == \
        ga.ATTN_ERR_NULL_ARG


def test_kv_cache_fp8_bytes(ga):
    g = _geom(ga, n_q_heads=24, n_kv_heads=2, max_tokens=200)     # tpad 256
    rc, n = ga.attn_kv_cache_fp8_bytes(g)
    assert rc == ga.ATTN_OK and n == 2 * 2 * 256 * 256 + 2 * 2 * 256 * 4
    rc, n = ga.attn_kv_cache_fp8_bytes(_geom(ga, n_q_heads=24, n_kv_heads=5))
    assert rc == ga.ATTN_ERR_GEOMETRY and n == 0
    assert ga.lib.attn_kv_cache_fp8_bytes(ctypes.byref(g), None) == ga.ATTN_ERR_NULL_ARG


WEIGHT_REFUSALS = [
    # (T, q_base, kind, mask, out, weights, expected)
    (64, 0, 4, FAKE, FAKE, FAKE, "RANGE"),         # cache kinds have no weights variant
    (256, 128, 5, FAKE, FAKE, FAKE, "RANGE"),
    (64, 0, 7, None, FAKE, FAKE, "RANGE"),
    (64, 0, -1, None, FAKE, FAKE, "RANGE"),
    (64, 0, 0, None, FAKE, None, "NULL_ARG"),      # weights missing
    (64, 0, 0, None, FAKE, FAKE + 8, "ALIGN"),     # weights misaligned
    (64, 0, 2, None, FAKE, FAKE, "NULL_ARG"),      # masked without a mask
    (64, 0, 0, None, None, FAKE, "NULL_ARG"),      # out missing
    (300, 0, 0, None, FAKE, FAKE, "RANGE"),        # T > max_tokens
    (200, 64, 1, None, FAKE, FAKE, "ALIGN"),       # q_base % 128
]


@pytest.mark.parametrize("case", WEIGHT_REFUSALS, ids=lambda c: f"{c[-1]}")
def test_weights_refusals(ga, case):
    T, qb, kind, mask, out, w, want = case
    rc = ga.attn_validate_weights(_geom(ga), _inputs(ga, 256), T, qb, kind, mask, out, w)
    assert rc == getattr(ga, "ATTN_ERR_" + want), (rc, ga.attn_status_string(rc))


def test_weights_valid_and_empty(ga):
    g, inp = _geom(ga), _inputs(ga, 256)
    for T, qb, kind, mask in [(256, 0, 0, None), (256, 128, 1, None), (256, 0, 2, FAKE + 3), (100, 0, 3, None)]:
        assert ga.attn_validate_weights(g, inp, T, qb, kind, mask, FAKE, FAKE) == ga.ATTN_OK
    # an empty window needs no pointers at all
    assert ga.attn_validate_weights(g, None, 0, 0, 0, None, None, None) == ga.ATTN_OK
    assert ga.attn_validate_weights(g, None, 128, 128, 1, None, None, None) == ga.ATTN_OK
    assert ga.lib.attn_validate_weights(None, None, 0, 0, 0, None, None, None) == ga.ATTN_ERR_NULL_ARG
    assert ga.attn_prefill_weights(None, inp, 64, 0, 0, None, FAKE, FAKE, None) == ga.ATTN_ERR_NULL_ARG


def test_one_hip_runtime_in_the_process():
    """Importing the binding (before anything else imports torch) leaves one
    HIP runtime mapped: the library must share torch's, whose device memory
    and streams it is handed.  Two runtimes in one process make the library's
    device calls fail on a GPU."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import gated_gqa_causal_amd\n"
            "import torch\n"
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(paths)); print(sorted(paths))\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.splitlines()[0] == "1", r.stdout


def test_noalloc_refusals_before_device_work(ga):
    """The allocation-free entry point refuses on the host, before any device
    call: past its scratch (n_kv_heads * round_up(S, 64) > 32768), past the
    geometry's max_tokens, bad geometry, null pointers; S == 0 is a no-op."""
    inp = _inputs(ga, n_pos=32768)
    g = _geom(ga, n_q_heads=16, n_kv_heads=4, max_tokens=32768)
    assert ga.attn_prefill_gated_noalloc(g, inp, 8193, FAKE, None) == ga.ATTN_ERR_RANGE
    g2 = _geom(ga, n_q_heads=8, n_kv_heads=8, max_tokens=32768)
    assert ga.attn_prefill_gated_noalloc(g2, inp, 4097, FAKE, None) == ga.ATTN_ERR_RANGE
    assert ga.attn_prefill_gated_noalloc(_geom(ga, max_tokens=256), inp, 257, FAKE, None) == ga.ATTN_ERR_RANGE
    assert ga.attn_prefill_gated_noalloc(_geom(ga, n_kv_heads=5), inp, 64, FAKE, None) == ga.ATTN_ERR_GEOMETRY
    assert ga.attn_prefill_gated_noalloc(_geom(ga), None, 64, FAKE, None) == ga.ATTN_ERR_NULL_ARG
    assert ga.attn_prefill_gated_noalloc(_geom(ga), inp, 64, None, None) == ga.ATTN_ERR_NULL_ARG
    assert ga.attn_prefill_gated_noalloc(_geom(ga), inp, 0, None, None) == ga.ATTN_OK


def test_test_hooks_only_in_the_test_build(ga):
    """The test hooks (csrc/test_hooks.h) are exported by the test build alone;
    the product library has none of them."""
    import ctypes
    prod = ctypes.CDLL(ga.LIBPATH)
    assert not hasattr(prod, "attn_debug_prepare") and not hasattr(prod, "attn_debug_fp8_encode")
    test = ctypes.CDLL(ga.LIBPATH.replace("libgatedattn.so", "libgatedattn_test.so"))
    src = open(os.path.join(ROOT, "gated_gqa_causal_amd", "csrc", "test_hooks.h")).read()
    hooks = sorted(set(re.findall(r"ATTN_EXPORT\s+[\w\s\*]*?\b(attn_\w+)\s*\(", src)))
    assert hooks == ["attn_debug_fp8_encode", "attn_debug_prepare"]
    for n in declared_functions() + hooks:
        assert hasattr(test, n), f"{n} not exported by the test build"
    f = test.attn_debug_prepare
    f.argtypes = [ctypes.c_void_p, ctypes.POINTER(ga.attn_inputs), ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, ctypes.byref(_inputs(ga)), 64, 0, FAKE, FAKE, None) == ga.ATTN_ERR_NULL_ARG
    g = test.attn_debug_fp8_encode
    g.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_void_p]
    assert g(FAKE, FAKE, FAKE, FAKE, -1, None) == ga.ATTN_ERR_RANGE
    assert g(FAKE, FAKE, FAKE, FAKE, (1 << 30) + 1, None) == ga.ATTN_ERR_RANGE
    assert g(None, FAKE, FAKE, FAKE, 16, None) == ga.ATTN_ERR_NULL_ARG
    assert g(FAKE, FAKE, FAKE, None, 16, None) == ga.ATTN_ERR_NULL_ARG
    assert g(None, None, None, None, 0, None) == ga.ATTN_OK
