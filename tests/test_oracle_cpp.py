"""Pins of the plain C++ float64 oracle (``oracle/ttt_oracle.cpp``).

The C++ oracle is a second, independent statement of the inner loop (it
shares no code with the numpy oracle or with the HIP path).  It is pinned the
four ways the method's description asks of an oracle, each against something
other than itself:

* its fast-weight gradients match central finite differences on tiny models
  to 1e-6 relative error (brute force);
* lr = 0 reproduces a plain sliding-window Transformer, here written with
  torch's own float64 library routines (layer_norm, scaled-dot-product
  attention with a band mask, gelu, silu, complex rotation, cross_entropy);
* a window covering the context reproduces full causal attention (torch's
  is_causal attention);
* per-chunk loss drops on planted repeated segments;

plus literal RoPE values, torch's attention on its own, and agreement with the
numpy oracle (itself pinned in test_oracle_pins.py) to float64 rounding on
every option: GELU and SwiGLU, several fast blocks, the frozen second MLP,
steps = 2, a ragged last chunk, a final chunk without target, positions past
5e5, and decode through decode-time updates.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import cpp
from oracle import ttt_oracle as O


def tiny_cfg(**kw):
    base = dict(name="pin", n_layers=3, d_model=16, n_heads=2, head_dim=8, d_ff=32, vocab=11,
                window=5, n_fast=2, mlp="gelu", dtype="fp32", T=24, chunk=8, lr=0.05, steps=1,
                seg=4, period=8, dmin=6, dmax=None, token_seed=7, weight_seed=77)
    base.update(kw)
    return synth.config(base)


def weights_std(cfg, std, seed=None):
    return [w.double() for w in synth.gen_weights(cfg, seed=seed, std=std)]


# ------------------------------------------------------- torch reference model

def _torch_rope(x, pos, base):
    """Rotate-half RoPE as a complex product: (x_i + i x_{i+hd/2}) e^{i p theta_i}."""
    n, H, hd = x.shape
    half = hd // 2
    theta = base ** (-2.0 * torch.arange(half, dtype=torch.float64) / hd)
    ang = pos.to(torch.float64)[:, None] * theta[None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def torch_swa_losses(cfg, w, x, window):
    """Per-position next-token losses of a plain pre-LN sliding-window
    Transformer with the loaded weights, from torch library routines."""
    d, H, hd = cfg["d_model"], cfg["n_heads"], cfg["head_dim"]
    eps, base = cfg["ln_eps"], cfg["rope_base"]
    names = synth.weight_names(cfg)
    W = dict(zip(names, [t.double() for t in w]))
    tok = torch.as_tensor(np.asarray(x), dtype=torch.long)
    n = len(tok)
    pos = torch.arange(n)
    band = (pos[None, :] <= pos[:, None]) & (pos[None, :] > pos[:, None] - window)

    def mlp(b, pre, l):
        if cfg["mlp"] == "gelu":
            return F.gelu(b @ W[f"L{l}.{pre}1"], approximate="none") @ W[f"L{l}.{pre}2"]
        return (F.silu(b @ W[f"L{l}.{pre}g"]) * (b @ W[f"L{l}.{pre}u"])) @ W[f"L{l}.{pre}d"]

    h = W["E"][tok]
    for l in range(cfg["n_layers"]):
        a = F.layer_norm(h, (d,), eps=eps)
        q = _torch_rope((a @ W[f"L{l}.Wq"]).view(n, H, hd), pos, base)
        k = _torch_rope((a @ W[f"L{l}.Wk"]).view(n, H, hd), pos, base)
        v = (a @ W[f"L{l}.Wv"]).view(n, H, hd)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                           attn_mask=band)
        h = h + o.transpose(0, 1).reshape(n, d) @ W[f"L{l}.Wo"]
        h = h + mlp(F.layer_norm(h, (d,), eps=eps), "W", l)
        if f"L{l}.S{'1' if cfg['mlp'] == 'gelu' else 'g'}" in W:
            h = h + mlp(F.layer_norm(h, (d,), eps=eps), "S", l)
    logits = F.layer_norm(h, (d,), eps=eps) @ W["U"]
    return F.cross_entropy(logits[:-1], tok[1:], reduction="none").numpy()


# ------------------------------------------------------------------ elements

def test_rope_literal_values_and_rotate_half_pairing():
    """theta_i = 10000^(-2i/hd): with hd = 8 at position 7 pair 1 turns by
    0.7 rad and pair 3 by 0.007 rad; e_0 goes to cos(1) e_0 + sin(1) e_4
    at position 1 (rotate-half), never into e_1; sign -1 undoes it."""
    x = np.zeros((1, 1, 8)); x[0, 0, 1] = 1.0
    y = cpp.rope(x, [7])[0, 0]
    assert abs(y[1] - math.cos(0.7)) < 1e-15 and abs(y[5] - math.sin(0.7)) < 1e-15
    x = np.zeros((1, 1, 8)); x[0, 0, 3] = 1.0
    y = cpp.rope(x, [7])[0, 0]
    assert abs(y[3] - math.cos(0.007)) < 1e-15 and abs(y[7] - math.sin(0.007)) < 1e-15
    e0 = np.zeros((1, 1, 8)); e0[0, 0, 0] = 1.0
    y = cpp.rope(e0, [1])[0, 0]
    ref = np.zeros(8); ref[0], ref[4] = math.cos(1.0), math.sin(1.0)
    np.testing.assert_allclose(y, ref, atol=1e-15)
    rng = np.random.default_rng(3)
    z = rng.normal(size=(5, 3, 16))
    p = [0, 3, 17, 500_000, 524_800]
    np.testing.assert_allclose(cpp.rope(cpp.rope(z, p), p, sign=-1), z, atol=1e-12)


def test_layer_norm_against_torch():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 7)) * 3 + 1
    ref = F.layer_norm(torch.tensor(x), (7,), eps=1e-5).numpy()
    np.testing.assert_allclose(cpp.layer_norm(x, 1e-5), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [1, 3, 6, 100])
def test_attention_against_torch_sdpa(window):
    """Library routine: torch's attention with the band mask, keys that
    include earlier (cached) positions before the queries."""
    rng = np.random.default_rng(window)
    nq, nc, H, hd = 7, 4, 2, 8
    q = rng.normal(size=(nq, H, hd)); k = rng.normal(size=(nc + nq, H, hd)); v = rng.normal(size=(nc + nq, H, hd))
    qpos = np.arange(nc, nc + nq); kpos = np.arange(nc + nq)
    o = cpp.attention(q, k, v, qpos, kpos, window)
    mask = torch.tensor((kpos[None, :] <= qpos[:, None]) & (kpos[None, :] > qpos[:, None] - window))
    ref = F.scaled_dot_product_attention(torch.tensor(q).transpose(0, 1), torch.tensor(k).transpose(0, 1),
                                         torch.tensor(v).transpose(0, 1), attn_mask=mask).transpose(0, 1)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------- the four self-checks

@pytest.mark.parametrize("n_fast,mlp,static", [(1, "gelu", 0), (2, "gelu", 0), (2, "swiglu", 0),
                                               (3, "swiglu", 0), (1, "swiglu", 1), (2, "gelu", 1)])
def test_fast_weight_gradient_finite_differences(n_fast, mlp, static):
    """Analytic gradient of the second chunk's loss (attention over cached
    keys that must stay constant) against central finite differences:
    largest and random entries of every fast matrix, and a random direction
    through all of them; relative error <= 1e-6."""
    cfg = tiny_cfg(n_fast=n_fast, mlp=mlp, static_mlp=static)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    C = cfg["chunk"]
    m = cpp.CppOracle(cfg, w)
    m.read(x[:C], 0, C)
    toks, tgt = x[C:2 * C], x[C + 1:2 * C + 1]
    base = m.fast_weights()
    loss, grads = m.chunk_loss_grad(toks, tgt, C)
    nm = m.n_mlp

    def loss_with(mats):
        for i, a in enumerate(mats):
            m.set_fast_weight(i // nm, i % nm, a)
        out = m.chunk_loss_grad(toks, tgt, C, grads=False)[0]
        for i, a in enumerate(base):
            m.set_fast_weight(i // nm, i % nm, a)
        return out

    rng = np.random.default_rng(5)
    h = 1e-5
    errs, mags = [], []
    for i, g in enumerate(grads):
        flat = np.argsort(-np.abs(g).ravel())[:6].tolist() + rng.integers(0, g.size, 4).tolist()
        for fi in flat:
            idx = np.unravel_index(fi, g.shape)
            plus = [a.copy() for a in base]; plus[i][idx] += h
            minus = [a.copy() for a in base]; minus[i][idx] -= h
            fd = (loss_with(plus) - loss_with(minus)) / (2 * h)
            errs.append(abs(fd - g[idx]))
            mags.append(abs(g[idx]))
    assert max(mags) > 1e-3
    assert max(errs) / max(mags) <= 1e-6, (max(errs), max(mags))
    dirs = [rng.normal(size=a.shape) for a in base]
    fd = (loss_with([a + h * d for a, d in zip(base, dirs)])
          - loss_with([a - h * d for a, d in zip(base, dirs)])) / (2 * h)
    an = sum(float((g * d).sum()) for g, d in zip(grads, dirs))
    assert abs(fd - an) / abs(an) <= 1e-6


@pytest.mark.parametrize("mlp,static", [("gelu", 0), ("swiglu", 0), ("swiglu", 1)])
def test_lr_zero_is_plain_swa_transformer(mlp, static):
    """lr = 0: the chunked loop's per-chunk losses equal the chunk means of
    a plain sliding-window Transformer built from torch's routines (ragged
    last chunk), and the fast weights do not move."""
    cfg = tiny_cfg(window=7, chunk=5, T=23, mlp=mlp, static_mlp=static)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    m = cpp.CppOracle(cfg, w)
    r = m.prefill(x, 5, 0.0)
    per = torch_swa_losses(cfg, w, x, 7)
    ref = [per[k * 5:min(k * 5 + 5, 22)].mean() for k in range(5)]
    np.testing.assert_allclose(r["losses"], ref, rtol=1e-12)
    names = synth.weight_names(cfg)
    fast_names = [n for n in names if n.startswith(tuple(f"L{l}.W" for l in range(1, 3)))
                  and n.split(".")[1] in ("W1", "W2", "Wg", "Wu", "Wd")]
    by = dict(zip(names, w))
    for a, n in zip(r["fast"], fast_names):
        assert np.array_equal(a, by[n].numpy())


def test_window_covering_context_is_full_causal_attention():
    """Window >= T at lr = 0 equals torch's is_causal attention model; with
    lr > 0 the result no longer depends on the window once it covers T."""
    cfg = tiny_cfg(T=24)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    r = cpp.prefill(synth.config(cfg, window=24), w, x, 8, 0.0)
    per = torch_swa_losses(cfg, w, x, 10**9)
    np.testing.assert_allclose(r["losses"], [per[0:8].mean(), per[8:16].mean(), per[16:23].mean()], rtol=1e-12)
    a = cpp.prefill(synth.config(cfg, window=24), w, x, 8, 0.05)
    b = cpp.prefill(synth.config(cfg, window=10**6), w, x, 8, 0.05)
    np.testing.assert_array_equal(a["losses"], b["losses"])
    c = cpp.prefill(synth.config(cfg, window=20), w, x, 8, 0.05)
    assert np.abs(c["losses"] - a["losses"]).max() > 0


def test_planted_repeats_lower_the_loss():
    """Tiny fp32 workload, T = 1024, lr 0.3: the update lowers the per-chunk
    loss below lr = 0, and lowers it more on chunks of planted copies (their
    sources beyond the window) than on fresh chunks."""
    cfg = synth.config("c1", T=1024)
    w = synth.gen_weights(cfg)
    x, copied = synth.gen_tokens(cfg, return_copies=True)
    C = cfg["chunk"]
    gain = cpp.prefill(cfg, w, x, C, 0.0)["losses"] - cpp.prefill(cfg, w, x, C, 0.3)["losses"]
    frac = np.array([copied[k * C + 1:(k + 1) * C + 1].mean() for k in range(len(gain))])
    late = np.arange(len(gain)) >= 8
    assert gain[late].mean() > 0
    assert gain[late & (frac > 0.5)].mean() > gain[late & (frac == 0)].mean()


# ------------------------------------------------- agreement with the numpy oracle

CASES = {
    "c1": lambda: (synth.config("c1"), None, 0),
    "swiglu-3fast": lambda: (tiny_cfg(mlp="swiglu", n_fast=3, T=29), 0.3, 0),
    "static-mlp": lambda: (tiny_cfg(mlp="gelu", static_mlp=1, T=30), 0.3, 0),
    "steps2": lambda: (tiny_cfg(steps=2, T=25), 0.3, 0),
    "target-less-last": lambda: (tiny_cfg(T=17), 0.3, 0),
    "far-positions": lambda: (tiny_cfg(mlp="swiglu", T=40, window=9), 0.3, 524_288),
    "chunk1": lambda: (tiny_cfg(chunk=1, T=12), 0.3, 0),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_agrees_with_numpy_oracle(case):
    cfg, std, off = CASES[case]()
    w = weights_std(cfg, std) if std else synth.gen_weights(cfg)
    x = synth.gen_tokens(cfg)
    C, lr, steps = cfg["chunk"], cfg["lr"], cfg["steps"]
    a = cpp.prefill(cfg, w, x, C, lr, steps, off)
    b = O.prefill(cfg, w, x, C, lr, steps, pos_offset=off)
    np.testing.assert_allclose(a["losses"], b["losses"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(a["last_logits"], b["last_logits"], rtol=1e-10, atol=1e-12)
    for p, q in zip(a["fast"], O.fast_weights_canonical(b)):
        np.testing.assert_allclose(p, q, rtol=1e-10, atol=1e-14)
        assert np.abs(p - q).max() <= 1e-10 * np.abs(q).max()


@pytest.mark.parametrize("forced", [True, False])
def test_decode_agrees_with_numpy_oracle(forced):
    """Tiny fp32 workload: prefill, then 40 decode positions through two
    decode-time updates (chunk 16), teacher-forced or greedy."""
    cfg = synth.config("c1")
    w = synth.gen_weights(cfg)
    x = synth.gen_tokens(cfg, T=cfg["T"] + 41)
    T = cfg["T"]
    m = cpp.CppOracle(cfg, w)
    m.prefill(x[:T], cfg["chunk"], cfg["lr"])
    st = O.prefill(cfg, w, x[:T], cfg["chunk"], cfg["lr"], return_state=True)
    f = x[T:T + 40] if forced else None
    a = m.decode(40, forced=f)
    b = O.decode(st, 40, forced=f)
    assert list(a["tokens"]) == list(b["tokens"])
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-10, atol=1e-12)
    assert len(a["update_losses"]) == 2
    np.testing.assert_allclose(a["update_losses"], b["update_losses"], rtol=1e-11)
    for p, q in zip(m.fast_weights(), O.fast_weights_canonical(st)):
        assert np.abs(p - q).max() <= 1e-10 * np.abs(q).max()
