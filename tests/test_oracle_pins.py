"""Pins of the float64 oracle against facts fixed by the pages and by
mathematics, independent of the oracle's own formulas.

Each test names the kind of pin: finite differences (brute force), a
library routine (torch's attention, scipy/math special functions), a closed
form, a special case or an invariant.  A plausible mistake in the oracle (a
dropped term, a wrong sign, a transposed operand, a wrong mask boundary, the
cache not held constant) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import ttt_oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def tiny_cfg(**kw):
    base = dict(name="pin", n_layers=3, d_model=16, n_heads=2, head_dim=8, d_ff=32, vocab=11,
                window=5, n_fast=2, mlp="gelu", dtype="fp32", T=24, chunk=8, lr=0.05, steps=1,
                seg=4, period=8, dmin=6, dmax=None, token_seed=7, weight_seed=77)
    base.update(kw)
    return synth.config(base)


def weights_std(cfg, std, seed=None):
    return [w.double() for w in synth.gen_weights(cfg, seed=seed, std=std)]


# ----------------------------------------------------------------- elements

def _fd(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp = x.copy(); xp[i] += h
        xm = x.copy(); xm[i] -= h
        g[i] = (f(xp) - f(xm)) / (2 * h)
    return g


def test_layer_norm_against_torch_and_fd():
    """Library routine (torch.layer_norm, no affine) + finite differences."""
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 7)) * 3 + 1
    y, rstd = O.layer_norm(x, 1e-5)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (7,), eps=1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    dy = rng.normal(size=(5, 7))
    dx = O.layer_norm_backward(dy, y, rstd)
    fd = _fd(lambda z: float((O.layer_norm(z, 1e-5)[0] * dy).sum()), x)
    np.testing.assert_allclose(dx, fd, rtol=1e-6, atol=1e-8)


def test_activations_against_math_and_fd():
    """GELU against math.erf (exact form), SiLU closed form, derivatives by FD."""
    z = np.linspace(-6, 6, 49)
    ref = np.array([0.5 * t * (1 + math.erf(t / math.sqrt(2))) for t in z])
    np.testing.assert_allclose(O.gelu(z), ref, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.silu(z), z * torch.sigmoid(torch.tensor(z)).numpy(), rtol=1e-13)
    h = 1e-6
    np.testing.assert_allclose(O.gelu_grad(z), (O.gelu(z + h) - O.gelu(z - h)) / (2 * h), rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(O.silu_grad(z), (O.silu(z + h) - O.silu(z - h)) / (2 * h), rtol=1e-7, atol=1e-9)


def test_rope_relative_position_and_transpose():
    """RoPE is a rotation: scores depend only on the position difference;
    norms are kept; the backward is the transpose of the forward."""
    rng = np.random.default_rng(1)
    hd = 8
    q = rng.normal(size=(1, 1, hd))
    k = rng.normal(size=(1, 1, hd))
    def score(pq, pk):
        cq, sq = O.rope_cos_sin(np.array([pq]), hd, 10000.0)
        ck, sk = O.rope_cos_sin(np.array([pk]), hd, 10000.0)
        return float((O.rope_apply(q, cq, sq) * O.rope_apply(k, ck, sk)).sum())
    assert abs(score(7, 3) - score(1007, 1003)) < 1e-11
    assert abs(score(7, 3) - score(3, 7)) > 1e-6          # not symmetric: positions matter
    x = rng.normal(size=(4, 2, hd))
    c, s = O.rope_cos_sin(np.arange(4) + 5, hd, 10000.0)
    y = O.rope_apply(x, c, s)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    dy = rng.normal(size=y.shape)
    assert abs((y * dy).sum() - (x * O.rope_backward(dy, c, s)).sum()) < 1e-12
    # position 0 is the identity; frequency 0 rotates by exactly the position
    c0, s0 = O.rope_cos_sin(np.array([0, 3]), hd, 10000.0)
    assert np.all(c0[0] == 1) and np.all(s0[0] == 0)
    assert abs(c0[1, 0] - math.cos(3.0)) < 1e-15


def test_rope_frequency_law_literal_values():
    """Closed form of the frequency law theta_i = base^(-2i/hd): with hd = 8
    and base 10000 the four pairs turn by 1, 0.1, 0.01 and 0.001 rad per
    position, so position 7 turns pair 1 by 0.7 rad and pair 3 by 0.007 rad;
    with hd = 4, pair 1 turns by 0.01 rad per position (0.05 rad at position
    5).  The expected cosines and sines are written out as numbers."""
    c, s = O.rope_cos_sin(np.array([7]), 8, 10000.0)
    assert abs(c[0, 0] - 0.7539022543433046) < 1e-15 and abs(s[0, 0] - 0.6569865987187891) < 1e-15
    assert abs(c[0, 1] - 0.7648421872844885) < 1e-15 and abs(s[0, 1] - 0.644217687237691) < 1e-15
    assert abs(c[0, 3] - 0.9999755001000415) < 1e-15 and abs(s[0, 3] - 0.006999942833473391) < 1e-15
    c4, s4 = O.rope_cos_sin(np.array([5]), 4, 10000.0)
    assert abs(c4[0, 1] - 0.9987502603949663) < 1e-15
    assert abs(s4[0, 1] - 0.04997916927067833) < 1e-15


def test_rope_rotate_half_pairing():
    """Rotate-half layout: component i is paired with i + hd/2 (an
    interleaved layout would pair 2i with 2i + 1).  With hd = 8: e_0 at
    position 1 becomes cos(1) e_0 + sin(1) e_4 and nothing else; e_5 (the
    second half of pair 1) at position 7 becomes cos(0.7) e_5 - sin(0.7) e_1;
    the backward (rotation by the negative angle) takes e_4 at position 1 to
    sin(1) e_0 + cos(1) e_4.  Values written out as numbers."""
    def unit(i):
        x = np.zeros((1, 1, 8))
        x[0, 0, i] = 1.0
        return x
    c1, s1 = O.rope_cos_sin(np.array([1]), 8, 10000.0)
    c7, s7 = O.rope_cos_sin(np.array([7]), 8, 10000.0)
    e = np.zeros(8); e[0] = 0.5403023058681398; e[4] = 0.8414709848078965
    np.testing.assert_allclose(O.rope_apply(unit(0), c1, s1)[0, 0], e, rtol=0, atol=1e-15)
    e = np.zeros(8); e[5] = 0.7648421872844885; e[1] = -0.644217687237691
    np.testing.assert_allclose(O.rope_apply(unit(5), c7, s7)[0, 0], e, rtol=0, atol=1e-15)
    e = np.zeros(8); e[0] = 0.8414709848078965; e[4] = 0.5403023058681398
    np.testing.assert_allclose(O.rope_backward(unit(4), c1, s1)[0, 0], e, rtol=0, atol=1e-15)


@pytest.mark.parametrize("window", [1, 3, 6, 100])
def test_window_attention_against_torch_sdpa(window):
    """Library routine: torch's scaled_dot_product_attention with an explicit
    band mask (t - W < j <= t), float64; also the cached-key offset case."""
    rng = np.random.default_rng(window)
    nq, ncache, H, hd = 9, 4, 3, 8
    q = rng.normal(size=(nq, H, hd))
    k = rng.normal(size=(ncache + nq, H, hd))
    v = rng.normal(size=(ncache + nq, H, hd))
    qpos = np.arange(ncache, ncache + nq) + 20
    kpos = np.arange(ncache + nq) + 20
    o, p = O.window_attention(q, k, v, qpos, kpos, window)
    mask = (kpos[None, :] <= qpos[:, None]) & (kpos[None, :] > qpos[:, None] - window)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q).transpose(0, 1), torch.tensor(k).transpose(0, 1),
        torch.tensor(v).transpose(0, 1), attn_mask=torch.tensor(mask)).transpose(0, 1).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    if window == 1:
        np.testing.assert_allclose(o, v[ncache:], rtol=1e-13, atol=1e-13)
    if window >= ncache + nq:   # full causal attention, the textbook special case
        ref2 = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q).transpose(0, 1), torch.tensor(k[ncache:]).transpose(0, 1),
            torch.tensor(v[ncache:]).transpose(0, 1), is_causal=True).transpose(0, 1).numpy()
        o2, _ = O.window_attention(q, k[ncache:], v[ncache:], qpos, kpos[ncache:], window)
        np.testing.assert_allclose(o2, ref2, rtol=1e-12, atol=1e-12)


def test_attention_backward_fd():
    rng = np.random.default_rng(3)
    nq, H, hd, W = 5, 2, 4, 3
    q, k, v = (rng.normal(size=(nq, H, hd)) for _ in range(3))
    pos = np.arange(nq)
    do = rng.normal(size=(nq, H, hd))
    _, p = O.window_attention(q, k, v, pos, pos, W)
    dq, dk, dv = O.window_attention_backward(do, q, k, v, p)
    f = lambda qq, kk, vv: float((O.window_attention(qq, kk, vv, pos, pos, W)[0] * do).sum())
    np.testing.assert_allclose(dq, _fd(lambda z: f(z, k, v), q), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(dk, _fd(lambda z: f(q, z, v), k), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(dv, _fd(lambda z: f(q, k, z), v), rtol=1e-6, atol=1e-9)


def test_cross_entropy_two_class_closed_form():
    """V = 2: the loss is the logistic loss softplus(z_other - z_target) and
    the gradient of the target logit is -(1 - sigmoid(margin)) / m."""
    rng = np.random.default_rng(4)
    z = rng.normal(size=(6, 2)) * 4
    y = np.array([0, 1, 1, 0, 1, 0])
    loss, g = O.cross_entropy(z, y[:5])
    margin = z[np.arange(5), y[:5]] - z[np.arange(5), 1 - y[:5]]
    assert abs(loss - np.mean(np.log1p(np.exp(-margin)))) < 1e-14
    np.testing.assert_allclose(g[np.arange(5), y[:5]], -(1 - 1 / (1 + np.exp(-margin))) / 5, rtol=1e-12)
    assert np.all(g[5] == 0)
    np.testing.assert_allclose(g[:5].sum(axis=1), 0, atol=1e-15)


# ---------------------------------------------------------- whole inner loop

@pytest.mark.parametrize("n_fast,mlp,static", [(1, "gelu", 0), (2, "gelu", 0), (2, "swiglu", 0),
                                               (3, "swiglu", 0), (1, "swiglu", 1), (2, "gelu", 1)])
def test_fast_weight_gradient_finite_differences(n_fast, mlp, static):
    """The central pin: analytic fast-weight gradient of a chunk loss vs
    central finite differences, relative error <= 1e-6.  The chunk is the
    second one, so attention sees cached keys that must stay constant
    (stop-gradient); n_fast >= 2 exercises the attention backward; static = 1
    puts the frozen second MLP after every fast one, so the gradient passes
    through it."""
    cfg = tiny_cfg(n_fast=n_fast, mlp=mlp, static_mlp=static)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    model = O.OracleModel(cfg, w)
    fast = model.initial_fast()
    C = cfg["chunk"]
    fw = O.forward_chunk(model, fast, O.empty_cache(cfg), x[:C], 0)
    cache = O._commit(cfg, O.empty_cache(cfg), fw, cfg["window"] + C)
    toks, tgt = x[C:2 * C], x[C + 1:2 * C + 1]
    loss, grads, _ = O.chunk_loss_and_grad(model, fast, cache, toks, tgt, C)

    def loss_at(fl, name, idx, delta):
        f2 = [{n: a.copy() for n, a in f.items()} for f in fast]
        f2[fl][name][idx] += delta
        return O.chunk_loss_and_grad(model, f2, cache, toks, tgt, C)[0]

    rng = np.random.default_rng(5)
    h = 1e-5
    errs, mags = [], []
    for fl in range(n_fast):
        for name, g in grads[fl].items():
            flat = np.argsort(-np.abs(g).ravel())[:6].tolist() + rng.integers(0, g.size, 4).tolist()
            for fi in flat:
                idx = np.unravel_index(fi, g.shape)
                fd = (loss_at(fl, name, idx, h) - loss_at(fl, name, idx, -h)) / (2 * h)
                errs.append(abs(fd - g[idx]))
                mags.append(abs(g[idx]))
    assert max(mags) > 1e-3
    assert max(errs) / max(mags) <= 1e-6, (max(errs), max(mags))

    # a random direction through all fast weights at once
    dirs = [{n: rng.normal(size=a.shape) for n, a in f.items()} for f in fast]
    def loss_dir(t):
        f2 = [{n: a + t * dirs[i][n] for n, a in f.items()} for i, f in enumerate(fast)]
        return O.chunk_loss_and_grad(model, f2, cache, toks, tgt, C)[0]
    fd = (loss_dir(h) - loss_dir(-h)) / (2 * h)
    an = sum(float((grads[i][n] * dirs[i][n]).sum()) for i in range(n_fast) for n in grads[i])
    assert abs(fd - an) / abs(an) <= 1e-6


@pytest.mark.parametrize("mlp", ["gelu", "swiglu"])
def test_zero_static_mlp_is_the_plain_block(mlp):
    """Special case: a frozen second MLP whose output projection is zero adds
    nothing, forward or backward, so losses and updated fast weights equal
    those of the blocks without it, exactly; with random weights it does
    change them, and it is never updated."""
    cfg = tiny_cfg(mlp=mlp)
    cfs = synth.config(cfg, static_mlp=1)
    w = weights_std(cfg, 0.3)
    ws = weights_std(cfs, 0.3)
    names, names_s = synth.weight_names(cfg), synth.weight_names(cfs)
    by = dict(zip(names, w))
    z = [by[n] if n in by else (torch.zeros_like(t) if n.endswith(("S2", "Sd")) else t)
         for n, t in zip(names_s, ws)]
    x = synth.gen_tokens(cfg)
    a = O.prefill(cfg, w, x, 8, 0.05)
    b = O.prefill(cfs, z, x, 8, 0.05)
    np.testing.assert_array_equal(a["losses"], b["losses"])
    for fa, fb in zip(a["fast"], b["fast"]):
        for n in fa:
            np.testing.assert_array_equal(fa[n], fb[n])
    r = [by[n] if n in by else t for n, t in zip(names_s, ws)]
    c = O.prefill(cfs, r, x, 8, 0.05, return_state=True)
    assert np.abs(c["losses"] - a["losses"]).max() > 1e-3
    for st, n in zip(c["model"].static, range(cfg["n_fast"])):
        l = cfg["n_layers"] - cfg["n_fast"] + n
        for k, arr in st.items():
            np.testing.assert_array_equal(arr, ws[names_s.index(f"L{l}.{k.replace('W', 'S')}")].numpy())


def test_lr_zero_is_plain_swa_forward():
    """lr = 0: chunked per-chunk losses equal the chunk means of one
    full-sequence forward (no chunks, no cache), and the fast weights are
    unchanged bit for bit.  Pins chunking, the cache and the window mask
    across chunk boundaries.  T is not a multiple of the chunk (ragged)."""
    cfg = tiny_cfg(window=7, chunk=5, T=23)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    r = O.prefill(cfg, w, x, 5, 0.0)
    per = O.sequence_forward_losses(cfg, w, x)
    ref = [per[k * 5:min(k * 5 + 5, 22)].mean() for k in range(5)]
    np.testing.assert_allclose(r["losses"], ref, rtol=1e-12)
    init = O.OracleModel(cfg, w).initial_fast()
    for a, b in zip(r["fast"], init):
        for n in a:
            assert np.array_equal(a[n], b[n])


def test_window_covering_context_is_full_attention():
    """Window >= T: the result does not depend on the window any more (full
    causal attention, whose kernel is pinned against the library)."""
    cfg = tiny_cfg(window=24)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    a = O.prefill(cfg, w, x, 8, 0.05)
    b = O.prefill(synth.config(cfg, window=10**6), w, x, 8, 0.05)
    np.testing.assert_array_equal(a["losses"], b["losses"])
    c = O.prefill(synth.config(cfg, window=20), w, x, 8, 0.05)
    assert np.abs(c["losses"] - a["losses"]).max() > 0     # a window below T does cut keys


def test_zero_head_gives_log_vocab_and_no_update():
    """U = 0: every logit is 0, so every loss is ln V exactly and the
    gradient (hence the update) is zero."""
    cfg = tiny_cfg()
    w = weights_std(cfg, 0.3)
    w[-1] = torch.zeros_like(w[-1])
    x = synth.gen_tokens(cfg)
    r = O.prefill(cfg, w, x, 8, 1.0)
    np.testing.assert_allclose(r["losses"], math.log(cfg["vocab"]), rtol=0, atol=1e-15)
    init = O.OracleModel(cfg, w).initial_fast()
    for a, b in zip(r["fast"], init):
        for n in a:
            assert np.array_equal(a[n], b[n])


def test_rope_shift_invariance_of_losses():
    """Shifting every absolute position by a constant leaves all losses and
    updates unchanged (RoPE only sees differences)."""
    cfg = tiny_cfg()
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    a = O.prefill(cfg, w, x, 8, 0.05)
    b = O.prefill(cfg, w, x, 8, 0.05, pos_offset=12345)
    np.testing.assert_allclose(a["losses"], b["losses"], rtol=1e-10)


def test_update_is_gradient_descent_first_order():
    """Two steps on one chunk: the second loss drops by lr*|g|^2 to first
    order ((l0 - l1) / (lr |g|^2) -> 1 as lr -> 0), with g from finite
    differences of the loss itself.  Pins the sign, the scale (mean, not
    sum) and that the update goes to the fast weights."""
    cfg = tiny_cfg(n_fast=2, T=8, chunk=8)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    model = O.OracleModel(cfg, w)
    _, grads, _ = O.chunk_loss_and_grad(model, model.initial_fast(), O.empty_cache(cfg),
                                        x[:8], x[1:8], 0)
    g2 = sum(float((g[n] ** 2).sum()) for g in grads for n in g)
    ratios = []
    for lr in (1e-3, 1e-4):
        r = O.prefill(cfg, w, x, 8, lr, steps=2)
        ratios.append((r["losses"][0] - r["losses"][1]) / (lr * g2))
    assert abs(ratios[-1] - 1) < 1e-3
    assert abs(ratios[-1] - 1) < abs(ratios[0] - 1) + 1e-12


def test_one_chunk_one_step_is_full_batch_gradient_step():
    """chunk = T, steps = 1: phi_1 = phi_0 - lr * grad of the mean loss,
    with the gradient taken by finite differences on a few entries."""
    cfg = tiny_cfg(n_fast=2, T=10, chunk=10)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    lr = 0.1
    r = O.prefill(cfg, w, x, 10, lr)
    model = O.OracleModel(cfg, w)
    f0 = model.initial_fast()
    h = 1e-5
    for fl, name, idx in [(0, "W1", (3, 5)), (1, "W2", (7, 2)), (1, "W1", (0, 0))]:
        def L(delta):
            f2 = [{n: a.copy() for n, a in f.items()} for f in f0]
            f2[fl][name][idx] += delta
            return O.chunk_loss_and_grad(model, f2, O.empty_cache(cfg), x, x[1:], 0)[0]
        g = (L(h) - L(-h)) / (2 * h)
        assert abs((f0[fl][name][idx] - r["fast"][fl][name][idx]) - lr * g) < 1e-9 * max(1.0, abs(lr * g))


def test_planted_repeats_lower_the_loss():
    """The update carries information beyond the window: with lr > 0 the
    per-chunk loss falls below the lr = 0 loss, and falls more on chunks
    made of planted copies (sources beyond the window) than on fresh ones.
    Workload: the tiny fp32 configuration at a larger lr (0.3) than its
    nominal 0.01, where the effect on random weights is clear of noise."""
    cfg = synth.config("c1", T=1024)
    w = synth.gen_weights(cfg)
    x, copied = synth.gen_tokens(cfg, return_copies=True)
    C = cfg["chunk"]
    r1 = O.prefill(cfg, w, x, C, 0.3)
    r0 = O.prefill(cfg, w, x, C, 0.0)
    gain = r0["losses"] - r1["losses"]
    frac = np.array([copied[k * C + 1:(k + 1) * C + 1].mean() for k in range(len(gain))])
    late = np.arange(len(gain)) >= 8
    rep = gain[late & (frac > 0.5)].mean()
    fresh = gain[late & (frac == 0)].mean()
    assert gain[late].mean() > 0
    assert rep > fresh, (rep, fresh)


def test_decode_teacher_forced_matches_prefill_logits():
    """lr = 0: decode positions read one at a time from the cache give the
    same logits as a one-shot forward of the concatenated sequence."""
    cfg = tiny_cfg(T=30)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    st = O.prefill(cfg, w, x[:20], 8, 0.0, return_state=True)
    d = O.decode(st, 10, forced=x[20:30])
    model = O.OracleModel(cfg, w)
    fw = O.forward_chunk(model, model.initial_fast(), O.empty_cache(cfg), x, 0)
    np.testing.assert_allclose(d["logits"], fw["logits"][20:30], rtol=1e-10, atol=1e-12)
    assert int(np.argmax(st["last_logits"] if st["last_logits"] is not None else fw["logits"][19])) >= 0


def test_decode_update_equals_prefill_chunk():
    """With lr > 0, a decode chunk (teacher-forced) makes exactly the update
    that reading those positions as one prefill chunk makes: same loss, same
    fast weights, same cache afterwards."""
    import copy
    cfg = tiny_cfg(T=32)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg, T=33)
    st = O.prefill(cfg, w, x[:24], 8, 0.05, return_state=True)
    model = st["model"]
    fast = copy.deepcopy(st["fast"])
    loss, grads, fw = O.chunk_loss_and_grad(model, fast, st["cache"], x[24:32], x[25:33], 24)
    d = O.decode(st, 8, forced=x[24:33])
    assert abs(d["update_losses"][0] - loss) < 1e-12
    for a, b, g in zip(st["fast"], fast, grads):
        for n in a:
            np.testing.assert_allclose(a[n], b[n] - 0.05 * g[n], rtol=1e-12, atol=1e-15)
    assert list(d["tokens"]) == list(x[24:32])


def test_greedy_argmax_ties_take_lowest_id():
    z = np.array([0.5, 2.0, 2.0, -1.0])
    assert int(np.argmax(z)) == 1


def test_steps_return_every_loss_and_commit_last_read():
    """steps = 2 returns two losses per chunk, the second after one update;
    steps = 1 with lr = 0 repeated twice gives the same loss twice."""
    cfg = tiny_cfg()
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    r = O.prefill(cfg, w, x, 8, 0.0, steps=2)
    assert len(r["losses"]) == 6
    np.testing.assert_array_equal(r["losses"][0::2], r["losses"][1::2])
    r2 = O.prefill(cfg, w, x, 8, 0.05, steps=2)
    assert np.all(r2["losses"][1::2] < r2["losses"][0::2])


def test_steps_two_keep_the_last_reads_keys_and_values():
    """steps = 2 built by hand from the pinned pieces: chunk 0 is read, the
    fast weights take one SGD step, chunk 0 is read again and takes a second
    step; the cache that chunk 1 attends to then holds the keys and values of
    the second read (they differ from the first read's above the lowest fast
    block, whose MLP changed in between).  The prefill's four losses equal
    this construction, and chunk 1's losses differ clearly from those of a
    cache built from the first read."""
    cfg = tiny_cfg(T=16, chunk=8, n_fast=2, window=12)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    lr = 0.05
    r = O.prefill(cfg, w, x, 8, lr, steps=2)
    model = O.OracleModel(cfg, w)
    empty = O.empty_cache(cfg)

    def step(fast, g):
        return [{n: f[n] - lr * gg[n] for n in f} for f, gg in zip(fast, g)]

    f0 = model.initial_fast()
    l00, g00, fw00 = O.chunk_loss_and_grad(model, f0, empty, x[:8], x[1:9], 0)
    f1 = step(f0, g00)
    l01, g01, fw01 = O.chunk_loss_and_grad(model, f1, empty, x[:8], x[1:9], 0)
    f2 = step(f1, g01)

    def cache_of(fw):
        return [(np.arange(8), fw["layers"][l]["k"], fw["layers"][l]["v"]) for l in range(cfg["n_layers"])]

    def chunk1(cache):
        l10, g10, _ = O.chunk_loss_and_grad(model, f2, cache, x[8:16], x[9:16], 8)
        l11 = O.chunk_loss_and_grad(model, step(f2, g10), cache, x[8:16], x[9:16], 8)[0]
        return l10, l11

    last, first = chunk1(cache_of(fw01)), chunk1(cache_of(fw00))
    np.testing.assert_allclose(r["losses"], [l00, l01, last[0], last[1]], rtol=1e-13)
    assert min(abs(last[0] - first[0]), abs(last[1] - first[1])) > 1e-6
    top = cfg["n_layers"] - 1
    assert np.abs(fw01["layers"][top]["k"] - fw00["layers"][top]["k"]).max() > 1e-6


def test_target_less_final_chunk():
    """T = 17, chunk 8: the third chunk holds only position 16, which has no
    target; it makes no update and reports 0."""
    cfg = tiny_cfg(T=17)
    w = weights_std(cfg, 0.3)
    x = synth.gen_tokens(cfg)
    r = O.prefill(cfg, w, x, 8, 0.05)
    r2 = O.prefill(cfg, w, x, 8, 0.05, max_chunks=2)
    assert len(r["losses"]) == 3 and r["losses"][2] == 0.0
    for a, b in zip(r["fast"], r2["fast"]):
        for n in a:
            assert np.array_equal(a[n], b[n])
