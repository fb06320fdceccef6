"""The model loaded without a workspace argument (ttt_model_load_static):
its device state lives in the library's static per-device array and no
device memory is allocated.  It runs the same kernels as a model loaded into
a caller's workspace, so its results must equal that model's bit for bit:
checked on two loads in a row, the second with a smaller configuration and
context (the array keeps the first model's contents, which the load must
clear).  A second static model on the same device is refused while the first
is alive, and a configuration larger than the array is refused."""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_lm_chunk_amd as T
    return T


def small_cfg(**kw):
    base = dict(name="small", n_layers=3, d_model=64, n_heads=2, head_dim=32, d_ff=128,
                vocab=256, window=48, n_fast=2, mlp="swiglu", dtype="bf16", T=100, chunk=32,
                lr=0.05, steps=1, seg=16, period=64, dmin=50, dmax=None, token_seed=12,
                weight_seed=112)
    base.update(kw)
    return synth.config(base)


def _run(T_, cfg, w, x, static):
    m = T_.Model(cfg, [t.cuda() for t in w], max_chunk=cfg["chunk"], static_workspace=static)
    losses = m.prefill(torch.from_numpy(x).cuda(), cfg["chunk"], cfg["lr"]).cpu()
    fw = [t.cpu() for t in m.fast_weights()]
    toks, logits = [], []
    for _ in range(cfg["chunk"] + 2):      # through one decode-time update
        t, lg, _ = m.decode_step(want_logits=True)
        toks.append(int(t.item()))
        logits.append(lg.cpu())
    return m, losses, fw, toks, torch.stack(logits)


def test_static_workspace_model_equals_workspace_model():
    T_ = _gpu()
    cases = [(synth.config("c1"), 0.02), (small_cfg(), 0.05)]   # the second is smaller
    for i, (cfg, std) in enumerate(cases):
        say(f"case static-workspace load {i}: {cfg['name']} dtype={cfg['dtype']} T={cfg['T']} "
            f"chunk={cfg['chunk']}")
        w = synth.gen_weights(cfg, std=std)
        x = synth.gen_tokens(cfg)
        ref, l0, f0, t0, g0 = _run(T_, cfg, w, x, static=False)
        ref.close()
        st, l1, f1, t1, g1 = _run(T_, cfg, w, x, static=True)
        assert st.workspace is None
        say(f"  losses equal {torch.equal(l0, l1)}, decode tokens equal {t0 == t1}")
        assert torch.equal(l0, l1)
        assert all(torch.equal(a, b) for a, b in zip(f0, f1))
        assert t0 == t1 and torch.equal(g0, g1)
        assert torch.isfinite(l1).all()
        with pytest.raises(T_.TTTError) as e:
            T_.Model(cfg, [t.cuda() for t in w], max_chunk=cfg["chunk"], static_workspace=True)
        assert e.value.status == -6
        st.close()
    # larger than the static array: refused before any weight is read
    c2 = synth.config("c2")
    dummy = [torch.zeros(8, dtype=torch.bfloat16, device="cuda") for _ in range(synth.n_weights(c2))]
    with pytest.raises(T_.TTTError) as e:
        T_.Model(c2, dummy, static_workspace=True)
    assert e.value.status == -7
