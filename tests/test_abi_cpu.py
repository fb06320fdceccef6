"""Host-side checks of the C ABI that need no GPU: the library loads, every
function declared in include/ttt.h is exported, configuration validation and
workspace sizing behave as documented, and argument errors come back as
status codes (no device work is enqueued by any of these calls)."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ttt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    import long_context_lm_chunk_amd as T
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(T.lib, n), n
    assert set(names) == set(T.EXPORTED)


def test_workspace_sizes_and_bounded_memory():
    import long_context_lm_chunk_amd as T
    c4 = T.workspace_bytes(T.config_from_dict(synth.config("c4")))
    c5 = T.workspace_bytes(T.config_from_dict(synth.config("c5")))
    # the KV rings are bounded by the window, not by the context length:
    # 128K and 512K contexts need the same workspace
    assert c4 == c5
    assert 10e9 < c4 < 40e9
    c1 = T.workspace_bytes(T.config_from_dict(synth.config("c1")))
    assert c1 < 100e6
    # the frozen second MLP adds its weights, their transposes and its
    # activations; a window of T = 131072 (full attention at 128K) grows the rings
    cs = T.workspace_bytes(T.config_from_dict(synth.config("c4", static_mlp=1)))
    assert c4 < cs < c4 + 4e9
    cf = T.workspace_bytes(T.config_from_dict(synth.config("c4", window=131072)))
    assert 60e9 < cf < 120e9


@pytest.mark.parametrize("field,value", [("head_dim", 48), ("n_fast", 0), ("vocab", 100),
                                         ("dtype", 7), ("mlp", 3), ("window", 0), ("d_ff", 100),
                                         ("max_chunk", 0), ("static_mlp", 2), ("window", (1 << 22) + 1)])
def test_config_validation(field, value):
    import long_context_lm_chunk_amd as T
    c = T.config_from_dict(synth.config("c1"))
    if field == "head_dim":
        c.head_dim, c.n_heads = 48, 1
        c.d_model = 48
    else:
        setattr(c, field, value)
    n = ctypes.c_size_t(0)
    rc = T.lib.ttt_workspace_bytes(ctypes.byref(c), ctypes.byref(n))
    assert rc == -2, (field, rc)
    assert T.lib.ttt_last_error()


@pytest.mark.parametrize("overrides", [
    dict(max_chunk=65536),                          # chunk logits: 65536 x 32000 bf16 = 4.2 GB
    dict(prefill_block=131072),                     # phase-A activations: 131072 x 8192 bf16
    dict(max_chunk=40000, prefill_block=40000),     # SwiGLU chunk rows: 40000 x 16384 bf16
    dict(dtype="fp32", max_chunk=20000),            # fp32 chunk logits: 20000 x 32000 x 4
])
def test_config_refuses_gemm_operands_beyond_2gib(overrides):
    """Matrix-product operands are read with 32-bit byte offsets: a shape
    whose operand would span more than 2^31 - 1 bytes is refused when the
    configuration is checked (nothing is allocated or launched), while the
    3B workload and its 64K-chunk variant with a small vocabulary pass."""
    import long_context_lm_chunk_amd as T
    cfg = synth.config("c4")
    blk = overrides.pop("prefill_block", 0)
    mc = overrides.pop("max_chunk", None)
    c = T.config_from_dict(synth.config(cfg, **overrides), max_chunk=mc, prefill_block=blk)
    n = ctypes.c_size_t(0)
    assert T.lib.ttt_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == -2
    assert b"2^31" in T.lib.ttt_last_error()
    ok = T.config_from_dict(cfg)
    assert T.lib.ttt_workspace_bytes(ctypes.byref(ok), ctypes.byref(n)) == 0
    small = T.config_from_dict(synth.config(cfg, vocab=4096, d_ff=4096), max_chunk=65536)
    assert T.lib.ttt_workspace_bytes(ctypes.byref(small), ctypes.byref(n)) == 0


def test_argument_errors_without_device_work():
    import long_context_lm_chunk_amd as T
    assert T.lib.ttt_prefill(None, None, 10, 4, 0.1, 1, None, None) == -1
    assert T.lib.ttt_decode_step(None, None, None, None, None) == -1
    assert T.lib.ttt_reset(None, None) == -1
    assert T.lib.ttt_fast_weight(None, 0, 0, None, 0, None) == -1
    assert T.lib.ttt_fast_weight_delta(None, 0, 0, None, 0, None) == -1
    assert T.lib.ttt_forward(None, None, 10, 4, None, None) == -1
    assert T.lib.ttt_prefill_many(None, 0, None, 10, 4, 0.1, 1, None, None) == -1
    one = (ctypes.c_void_p * 1)(None)
    assert T.lib.ttt_prefill_many(one, 1, one, 10, 4, 0.1, 1, one, None) == -1   # a NULL handle
    c = T.config_from_dict(synth.config("c1"))
    h = ctypes.c_void_p(0)
    assert T.lib.ttt_model_load(ctypes.byref(c), None, 0, None, 0, None, ctypes.byref(h)) == -1
    assert T.lib.ttt_diag_gemm(1, 1, 1, 4, 4, 4, None, 8, None, 8, None, 8, None) == -1
    # output width / stride not a multiple of 4: rejected before any launch
    # (the pointers are never touched on this path)
    dummy = ctypes.c_void_p(4096)
    assert T.lib.ttt_diag_gemm(1, 1, 1, 4, 6, 8, dummy, 8, dummy, 8, dummy, 6, None) == -1
    assert T.lib.ttt_diag_gemm(1, 1, 1, 4, 8, 8, dummy, 8, dummy, 8, dummy, 6, None) == -1
    # the core selector only takes 0, 1, 2 and reports the mode in force
    mode = T.lib.ttt_diag_gemm_core(7)
    assert mode in (0, 1, 2) and T.lib.ttt_diag_gemm_core(7) == mode
    assert T.lib.ttt_status_str(-4) == b"token id out of range"
    T.lib.ttt_model_free(None)
