"""Parity at the full 3B shape, in the launch configuration of the timed
prefill: 28 layers, d 3072, 24 heads of 128, SwiGLU 8192, vocabulary 32000,
window 8192, the MLPs of the last 7 blocks fast, chunk 1024, lr 1e-4, bf16
storage, frozen blocks batched over 8192 tokens, a 131072-token context.

The float64 oracle cannot run the whole context (hours on the host), so the
outputs it can compute one by one are sampled: the first two chunk losses of
the full-context prefill (they depend only on tokens 0..2048 and on the
update made after chunk 0), and, from a 2048-token prefill in the same
configuration, both chunk losses, every fast matrix after the two updates
and the logits of three greedy decode positions; the same 2048-token case
also runs in the float32 check mode (bar 1e-4).  The rest of the 131072
positions are checked by properties: every chunk loss is finite, and the
first two agree with the 2048-token run.

The context read without updates (the static-weight model) is checked the
same way, at window 8192 and with full attention (window = T = 131072):
chunk 0 against the oracle, every chunk against the prefill at lr = 0
(window 8192), and the first 8 chunks of the two windows against each other
(no query before position 8192 has more keys than either window holds).
"""
import math
import sys

import numpy as np
import pytest
import torch

import synth
from greedy import greedy_ok
from oracle import ttt_oracle as O

pytestmark = pytest.mark.gpu

BAR = 2e-2   # bf16 storage, fp32 accumulation
_REF = {}    # oracle values shared by the tests of this module


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module")
def c4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_lm_chunk_amd as T_
    cfg = synth.config("c4")
    say("case 3B shape: weights and model load")
    w = synth.gen_weights(cfg, device="cuda:0")
    x = synth.gen_tokens(cfg)
    m = T_.Model(cfg, w, max_chunk=cfg["chunk"])
    yield cfg, w, x, m
    m.close()


@pytest.mark.timeout(1200)
def test_3b_full_context_first_chunks_weights_and_decode_match_oracle(c4):
    cfg, w, x, m = c4
    C, lr = cfg["chunk"], cfg["lr"]
    T = cfg["T"]
    tok = torch.from_numpy(x).cuda()

    say(f"case 3B full-context prefill T={T} chunk={C} lr={lr}")
    full = m.prefill(tok, C, lr).cpu().numpy()
    torch.cuda.synchronize()
    assert full.shape == (T // C,)
    assert np.all(np.isfinite(full))

    say("case 3B prefill T=2048, fast weights, 3 decode positions")
    two = m.prefill(tok[:2048], C, lr).cpu().numpy()
    fw = [t.cpu().numpy() for t in m.fast_weights()]
    fd = [t.cpu().numpy() for t in m.fast_weights(delta=True)]
    toks, logits = [], []
    for _ in range(3):
        t, lg, _ = m.decode_step(want_logits=True)
        toks.append(int(t.item()))
        logits.append(lg.cpu().numpy())
    torch.cuda.synchronize()

    say("case 3B fp32 check mode (the same bf16 values held as float32): prefill T=2048, "
        "fast weights, 3 decode positions")
    import long_context_lm_chunk_amd as T_
    m32 = T_.Model(cfg, [t.float() for t in w], dtype="fp32", max_chunk=C)
    two32 = m32.prefill(tok[:2048], C, lr).cpu().numpy()
    fw32 = [t.cpu().numpy() for t in m32.fast_weights()]
    fd32 = [t.cpu().numpy() for t in m32.fast_weights(delta=True)]
    toks32, logits32 = [], []
    for _ in range(3):
        t, lg, _ = m32.decode_step(want_logits=True)
        toks32.append(int(t.item()))
        logits32.append(lg.cpu().numpy())
    torch.cuda.synchronize()
    m32.close()
    del m32

    say("case 3B oracle: two chunks of 1024 and three decode positions (float64, host)")
    model = O.OracleModel(cfg, [t.cpu() for t in w], frozen_dtype=np.float32)
    st = O.prefill(cfg, None, x[:2048], C, lr, model=model, return_state=True)
    ref = st["losses"]
    _REF["loss0"] = float(ref[0])   # chunk 0's loss is read before any update
    w0 = [a for f in st["model"].initial_fast() for a in f.values()]
    rfw = O.fast_weights_canonical(st)
    # decode leaves the prefill state's cache and weights as they were (no
    # update within 3 positions; the cache list is replaced, not modified)
    d = O.decode(dict(st), 3, forced=np.array(toks + [int(np.argmax(logits[-1]))]))
    d32 = O.decode(dict(st), 3, forced=np.array(toks32 + [int(np.argmax(logits32[-1]))]))

    e_two = float(np.max(np.abs(two - ref) / np.abs(ref)))
    e_full = float(np.max(np.abs(full[:2] - ref) / np.abs(ref)))
    e_w = max(rel(a, b) for a, b in zip(fw, rfw))
    e_dw = max(rel(a, b - c) for a, b, c in zip(fd, rfw, w0))
    e_dwm = max(float(np.abs(a - (b - c)).max() / np.abs(b - c).max()) for a, b, c in zip(fd, rfw, w0))
    say("  dW per matrix (Frobenius, max/max): " + " ".join(
        f"{rel(a, b - c):.1e}/{np.abs(a - (b - c)).max() / np.abs(b - c).max():.1e}"
        for a, b, c in zip(fd, rfw, w0)))
    L = np.array(logits)
    e_lg = float(np.abs(L - d["logits"]).max() / np.abs(d["logits"]).max())
    say(f"  errors: losses(T=2048) {e_two:.2e} losses(full, chunks 0-1) {e_full:.2e} "
        f"W {e_w:.2e} dW {e_dw:.2e} decode logits {e_lg:.2e}; "
        f"full vs 2048 run {np.max(np.abs(full[:2] - two) / np.abs(two)):.2e}")
    assert e_two < BAR and e_full < BAR and e_w < BAR and e_lg < BAR
    assert e_dwm < BAR
    e32 = dict(loss=float(np.max(np.abs(two32 - ref) / np.abs(ref))),
               W=max(rel(a, b) for a, b in zip(fw32, rfw)),
               dW=max(float(np.abs(a - (b - c)).max() / np.abs(b - c).max()) for a, b, c in zip(fd32, rfw, w0)),
               logits=float(np.abs(np.array(logits32) - d32["logits"]).max() / np.abs(d32["logits"]).max()))
    say("  fp32 check mode errors: " + ", ".join(f"{k} {v:.2e}" for k, v in e32.items()))
    assert e32["loss"] < 1e-4 and e32["W"] < 1e-4 and e32["logits"] < 1e-4
    assert e32["dW"] < 1e-4
    # the two GPU runs compute the same first two chunks
    np.testing.assert_allclose(full[:2], two, rtol=1e-3)
    # greedy tokens: the oracle's argmax where its top-2 gap is clear, a
    # near-tie elsewhere
    assert greedy_ok(toks[0], st["last_logits"], BAR)
    for i in range(2):
        assert greedy_ok(toks[i + 1], d["logits"][i], BAR)


@pytest.mark.timeout(1200)
def test_3b_decode_time_update_matches_oracle(c4):
    """A decode-time update at the 3B shape in bf16: a one-chunk prefill (1024
    tokens), then 1024 greedy decode positions; their completed chunk makes
    the same update as a prefill chunk would.  The oracle replays the emitted
    tokens (teacher forcing) as that chunk, read after the prefill state with
    the weights of that time (a decode chunk's update equals the prefill
    chunk's, pinned on the oracle by test_decode_update_equals_prefill_chunk).
    Compared: the logits of every position of both chunks as the chunk path
    kept them, the decode path's logits at several positions, the update's
    loss, and the change of every fast matrix (element-wise) after the
    prefill chunk and after the decode chunk."""
    cfg, w, x, m = c4
    C, lr = cfg["chunk"], cfg["lr"]
    tok = torch.from_numpy(x).cuda()
    say(f"case 3B decode-time update: prefill T={C}, then {C} greedy decode positions (one update)")
    m.prefill(tok[:C], C, lr)
    lg_pre = m.chunk_logits().cpu().numpy()
    fd_pre = [t.cpu().numpy() for t in m.fast_weights(delta=True)]
    keep = (0, 1, 511, C - 2, C - 1)
    toks, lgs, upd = [], {}, []
    for i in range(C):
        t, lg, ul = m.decode_step(want_logits=i in keep)
        toks.append(int(t.item()))
        if lg is not None:
            lgs[i] = lg.cpu().numpy().astype(np.float64)
        upd.append(float(ul.item()))
    lg_dec_chunk = m.chunk_logits().cpu().numpy()
    fd = [t.cpu().numpy() for t in m.fast_weights(delta=True)]
    torch.cuda.synchronize()
    say("case 3B decode-time update: oracle, prefill chunk and the decode chunk (float64, host)")
    model = O.OracleModel(cfg, [t.cpu() for t in w], frozen_dtype=np.float32)
    f0 = model.initial_fast()
    l0, g0, fw0 = O.chunk_loss_and_grad(model, f0, O.empty_cache(cfg), x[:C], x[1:C], 0)
    f1 = [{n: f[n] - lr * g[n] for n in f} for f, g in zip(f0, g0)]
    cache = O._commit(cfg, O.empty_cache(cfg), fw0, cfg["window"] + C)
    e = np.array(toks + [int(np.argmax(lgs[C - 1]))])
    loss, g1, fw1 = O.chunk_loss_and_grad(model, f1, cache, e[:C], e[1:], C)

    def rowerr(a, b):   # per row: max |a - b| / max |b|
        return np.abs(a - b).max(axis=1) / np.abs(b).max(axis=1)

    def dwerr(got, ref):
        return [float(np.abs(a - b).max() / np.abs(b).max()) for a, b in zip(got, ref)]

    names = model.mlp_names                                           # canonical order
    r_pre = [lr * -g[n] for g in g0 for n in names]                   # change by the prefill chunk
    r_dec = [lr * -g[n] for g in g1 for n in names]                   # change by the decode chunk
    e_pre = dwerr(fd_pre, r_pre)
    e_dec = dwerr([a - b for a, b in zip(fd, fd_pre)], r_dec)          # this update's own change
    e_tot = dwerr(fd, [a + b for a, b in zip(r_pre, r_dec)])
    er_pre = rowerr(lg_pre.astype(np.float64), fw0["logits"])
    er_dch = rowerr(lg_dec_chunk.astype(np.float64), fw1["logits"])
    e_lg = max(float(np.abs(lgs[i] - fw1["logits"][i]).max() / np.abs(fw1["logits"][i]).max()) for i in keep)
    e_lg_chunk_keep = max(float(er_dch[i]) for i in keep)
    got = [u for u in upd if not np.isnan(u)]
    e_loss = abs(got[0] - loss) / abs(loss)
    say(f"  chunk-path logits, prefill chunk: per-row max/max median {np.median(er_pre):.2e} worst "
        f"{er_pre.max():.2e}; decode chunk re-read: median {np.median(er_dch):.2e} worst {er_dch.max():.2e}")
    say(f"  decode-path logits at {keep}: {e_lg:.2e} (chunk path at the same positions {e_lg_chunk_keep:.2e})")
    say(f"  update loss {e_loss:.2e} ({got[0]:.6f} vs {loss:.6f})")
    say("  dW max/max per matrix, prefill chunk: " + " ".join(f"{v:.1e}" for v in e_pre))
    say("  dW max/max per matrix, decode chunk:  " + " ".join(f"{v:.1e}" for v in e_dec))
    say(f"  dW max/max worst: prefill chunk {max(e_pre):.2e}, decode chunk {max(e_dec):.2e}, "
        f"both {max(e_tot):.2e}")
    assert len(got) == 1 and not np.isnan(upd[C - 1])
    assert e_loss < BAR
    # the decode path rounds at the same points as the chunk path: its logits
    # are held to the bar, or to the chunk path's own error at the same
    # positions where bf16 at this depth already exceeds it
    assert e_lg < max(BAR, 1.25 * e_lg_chunk_keep)
    assert max(e_tot) < BAR
    assert greedy_ok(toks[0], fw0["logits"][-1], BAR)


@pytest.mark.timeout(1200)
def test_3b_512k_decode_time_update_equals_prefill_of_the_same_tokens(c4):
    """The 512K-context workload at its own size (the C4 weights, 524288
    context tokens, positions past 2^19), by a property the oracle cannot
    reach there: after the 512-chunk prefill, 1024 greedy decode positions
    make one decode-time update, and a prefill of the context followed by
    the emitted tokens makes, for its chunk 512, the same update (the
    decode-time update equals a prefill chunk's, pinned on the oracle by
    test_decode_update_equals_prefill_chunk).  The two runs share chunks
    0-510 bit for bit; chunk 511 has one target more in the longer run (the
    context's last position predicts the first emitted token there, and has
    no target at the end of the context), which moves that chunk's update
    by about 1/1024 of itself; beyond that they differ only in how the
    frozen layers read the decode chunk (matrix-vector products during
    decode, batched products in the prefill).  So the update's loss and its
    own change of every fast matrix must agree to the bf16 bar."""
    cfg5 = synth.config("c5")
    cfg, w, x_unused, m = c4
    C, lr, T = cfg["chunk"], cfg["lr"], cfg5["T"]
    x = synth.gen_tokens(cfg5)
    tok = torch.from_numpy(x).cuda()
    say(f"case 3B 512K: prefill T={T}, then {C} greedy decode positions (one decode-time update)")
    la = m.prefill(tok[:T], C, lr).cpu().numpy()
    fd_pre = m.fast_weights(delta=True)
    toks, upd, last = [], [], None
    for i in range(C):
        t, lg, ul = m.decode_step(want_logits=i == C - 1)
        toks.append(int(t.item()))
        upd.append(float(ul.item()))
        if lg is not None:
            last = int(torch.argmax(lg).item())
    fd_a = m.fast_weights(delta=True)
    got = [u for u in upd if not math.isnan(u)]
    say(f"case 3B 512K: prefill of the context and the {C + 1} emitted tokens (T={T + C + 1})")
    y = torch.cat([tok[:T], torch.tensor(toks + [last], dtype=torch.int32, device="cuda")])
    lb = m.prefill(y, C, lr).cpu().numpy()
    fd_b = m.fast_weights(delta=True)
    e_dw = [float(((a - p0) - (b - p0)).abs().max() / (b - p0).abs().max())
            for a, b, p0 in zip(fd_a, fd_b, fd_pre)]
    e_loss = abs(got[0] - lb[T // C]) / abs(lb[T // C])
    same = bool(np.array_equal(la[:T // C - 1], lb[:T // C - 1]))
    say(f"  update loss {got[0]:.6f} vs prefill chunk {T // C} {lb[T // C]:.6f}: {e_loss:.2e}; "
        f"chunk losses 0-{T // C - 2} equal: {same}; chunk {T // C - 1}: {la[-1]:.6f} (1023 targets) "
        f"vs {lb[T // C - 1]:.6f} (1024)")
    say("  the update's own dW max/max per matrix: " + " ".join(f"{v:.1e}" for v in e_dw))
    assert np.all(np.isfinite(la)) and same
    assert len(got) == 1 and not math.isnan(upd[C - 1])
    assert lb[T // C + 1] == 0.0                       # the last chunk has no target
    assert e_loss < BAR
    assert max(e_dw) < BAR


def _oracle_loss0(cfg, w, x):
    if "loss0" not in _REF:
        say("case 3B oracle: chunk 0 forward (float64, host)")
        per = O.sequence_forward_losses(cfg, [t.cpu() for t in w], x[:cfg["chunk"] + 1],
                                        frozen_dtype=np.float32)
        _REF["loss0"] = float(per.mean())
    return _REF["loss0"]


@pytest.mark.timeout(1200)
def test_3b_forward_without_updates_and_full_attention(c4):
    import long_context_lm_chunk_amd as T_
    cfg, w, x, m = c4
    C, T = cfg["chunk"], cfg["T"]
    tok = torch.from_numpy(x).cuda()
    say(f"case 3B forward without updates, window {cfg['window']}, T={T}")
    fw = m.forward(tok, C).cpu().numpy()
    p0 = m.prefill(tok, C, 0.0).cpu().numpy()
    torch.cuda.synchronize()
    assert np.all(np.isfinite(fw))
    say(f"  forward vs prefill(lr=0): {np.max(np.abs(fw - p0) / np.abs(p0)):.2e}")
    np.testing.assert_allclose(fw, p0, rtol=1e-3)

    say(f"case 3B full attention: window = T = {T}, forward and 2 decode positions")
    fa = T_.Model(synth.config(cfg, window=T), w, max_chunk=C)
    ffa = fa.forward(tok, C).cpu().numpy()
    dec = []
    for _ in range(2):
        t, lg, ul = fa.decode_step(want_logits=True)
        dec.append((int(t.item()), bool(torch.isfinite(lg).all().item()), float(ul.item())))
    torch.cuda.synchronize()
    fa.close()
    del fa
    assert np.all(np.isfinite(ffa))
    say(f"  full vs window-8192 forward, chunks 0-7: {np.max(np.abs(ffa[:8] - fw[:8]) / np.abs(fw[:8])):.2e}")
    np.testing.assert_allclose(ffa[:8], fw[:8], rtol=1e-3)
    for t, fin, ul in dec:
        assert 0 <= t < cfg["vocab"] and fin and np.isnan(ul)

    l0 = _oracle_loss0(cfg, w, x)
    e = max(abs(fw[0] - l0), abs(ffa[0] - l0)) / l0
    say(f"  chunk 0 vs oracle: {e:.2e}")
    assert e < BAR


@pytest.mark.timeout(1200)
def test_3b_static_second_mlp_first_chunks_match_oracle():
    """The variant whose 7 fast blocks also carry a frozen second MLP, at the
    3B shape in the same launch configuration: a 2048-token prefill (two
    chunks of 1024, frozen blocks batched over 8192) against the oracle,
    losses, fast matrices and their exact changes."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_lm_chunk_amd as T_
    cfg = synth.config("c4", static_mlp=1)
    C, lr = cfg["chunk"], cfg["lr"]
    say("case 3B static second MLP: prefill T=2048")
    w = synth.gen_weights(cfg, device="cuda:0")
    x = synth.gen_tokens(cfg, T=2048)
    m = T_.Model(cfg, w, max_chunk=C)
    got = m.prefill(torch.from_numpy(x).cuda(), C, lr).cpu().numpy()
    fw = [t.cpu().numpy() for t in m.fast_weights()]
    fd = [t.cpu().numpy() for t in m.fast_weights(delta=True)]
    torch.cuda.synchronize()
    m.close()
    say("case 3B static second MLP: oracle, two chunks (float64, host)")
    model = O.OracleModel(cfg, [t.cpu() for t in w], frozen_dtype=np.float32)
    del w
    st = O.prefill(cfg, None, x, C, lr, model=model, return_state=True)
    rfw = O.fast_weights_canonical(st)
    w0 = [a for f in st["model"].initial_fast() for a in f.values()]
    e_l = float(np.max(np.abs(got - st["losses"]) / np.abs(st["losses"])))
    e_w = max(rel(a, b) for a, b in zip(fw, rfw))
    e_dw = max(rel(a, b - c) for a, b, c in zip(fd, rfw, w0))
    e_dwm = max(float(np.abs(a - (b - c)).max() / np.abs(b - c).max()) for a, b, c in zip(fd, rfw, w0))
    say(f"  errors: losses {e_l:.2e} W {e_w:.2e} dW {e_dw:.2e} dW(max/max) {e_dwm:.2e}")
    assert e_l < BAR and e_w < BAR and e_dwm < BAR
