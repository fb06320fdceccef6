"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Every test runs the library's kernels on the GPU and the oracle on the CPU
on the same seeded inputs.  Relative errors (the checks of the inner loop):
  losses:        max_k |l_k - l*_k| / |l*_k|
  fast weights:  ||W - W*||_F / ||W*||_F for every fast matrix
  dW:            max |dW - dW*| / max |dW*| per fast matrix, element by
                 element, with dW = W - W0 read from the library's exact
                 float32 master of the change (W itself is dominated by W0)
Bars: 1e-4 in the float32 check mode, 2e-2 with bf16 storage, for all three.
Also asserted as a diagnostic:
  dloss: the loss change caused by the updates, (l(lr) - l(0)) vs oracle.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import cpp
from oracle import ttt_oracle as O

pytestmark = pytest.mark.gpu

BAR = {"fp32": 1e-4, "bf16": 2e-2}
# The loss change caused by the updates, l(lr) - l(0), is a difference of two
# numbers near ln V, so its relative error is the loss error magnified by
# |l| / |l(lr) - l(0)| (10^2 to 10^3 here); a diagnostic, with a bar of its own.
DLOSS_BAR = {"fp32": 1e-3, "bf16": 5e-2}
# Models up to this width are also checked against the plain C++ oracle.
CPP_ORACLE_MAX_D = 256


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_lm_chunk_amd as T
    return T


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def small_cfg(**kw):
    base = dict(name="small", n_layers=3, d_model=64, n_heads=2, head_dim=32, d_ff=128,
                vocab=256, window=48, n_fast=2, mlp="swiglu", dtype="fp32", T=200, chunk=32,
                lr=0.05, steps=1, seg=16, period=64, dmin=50, dmax=None, token_seed=11,
                weight_seed=111)
    base.update(kw)
    return synth.config(base)


def run_pair(cfg, dtype=None, std=0.02, T=None, chunk=None, lr=None, steps=1, prefill_block=0,
             lr0_too=True):
    """GPU prefill and oracle prefill on the same inputs; returns errors."""
    T_ = _gpu()
    dtype = dtype or cfg["dtype"]
    if dtype == "bf16":
        # bf16 runs draw bf16-rounded weights, so both sides see the same values
        cfg = synth.config(cfg, dtype="bf16")
    T = T or cfg["T"]
    chunk = chunk or cfg["chunk"]
    lr = cfg["lr"] if lr is None else lr
    say(f"case {cfg['name']} dtype={dtype} T={T} chunk={chunk} lr={lr} steps={steps} "
        f"L={cfg['n_layers']} d={cfg['d_model']} hd={cfg['head_dim']} q={cfg['n_fast']} {cfg['mlp']}")
    w = synth.gen_weights(cfg, std=std, device="cpu")
    if dtype == "fp32":
        w = [t.float() for t in w]
    x = synth.gen_tokens(cfg, T=T)
    m = T_.Model(cfg, [t.cuda() for t in w], dtype=dtype, max_chunk=chunk, prefill_block=prefill_block)
    tok = torch.from_numpy(x).cuda()
    losses = m.prefill(tok, chunk, lr, steps).cpu().numpy()
    fw = [t.cpu().numpy() for t in m.fast_weights()]
    fd = [t.cpu().numpy() for t in m.fast_weights(delta=True)]
    ref = O.prefill(cfg, w, x, chunk, lr, steps)
    rfw = O.fast_weights_canonical(ref)
    model0 = O.OracleModel(cfg, w)
    w0 = [a for f in model0.initial_fast() for a in f.values()]

    def errors(ref_losses, ref_fw):
        return dict(
            loss=float(np.max(np.abs(losses - ref_losses) / np.maximum(np.abs(ref_losses), 1e-12))),
            W=max(rel(a, b) for a, b in zip(fw, ref_fw)),
            dW=max(rel(a, b - c) for a, b, c in zip(fd, ref_fw, w0)),
            dWmax=max(float(np.abs(a - (b - c)).max() / max(np.abs(b - c).max(), 1e-300))
                      for a, b, c in zip(fd, ref_fw, w0)))

    out = errors(ref["losses"], rfw)
    if cfg["d_model"] <= CPP_ORACLE_MAX_D:
        # the plain C++ oracle too: each error is the larger of the two
        cref = cpp.prefill(cfg, w, x, chunk, lr, steps)
        ce = errors(cref["losses"], cref["fast"])
        say(f"  C++ oracle: loss {ce['loss']:.2e} W {ce['W']:.2e} dW(max/max) {ce['dWmax']:.2e}")
        out = {k: max(out[k], ce[k]) for k in out}
    out.update(losses=losses, ref=ref["losses"], model=m, w=w, x=x)
    if lr0_too:
        l0 = m.prefill(tok, chunk, 0.0, steps).cpu().numpy()
        r0 = O.prefill(cfg, w, x, chunk, 0.0, steps)["losses"]
        dg, dr = losses - l0, ref["losses"] - r0
        out["dloss"] = float(np.linalg.norm(dg - dr) / max(np.linalg.norm(dr), 1e-300))
        out["loss0"] = float(np.max(np.abs(l0 - r0) / np.maximum(np.abs(r0), 1e-12)))
    say(f"  errors: loss {out['loss']:.2e} W {out['W']:.2e} dW {out['dW']:.2e} dW(max/max) {out['dWmax']:.2e} "
        f"dloss {out.get('dloss', float('nan')):.2e} loss(lr=0) {out.get('loss0', float('nan')):.2e}")
    return out


# ------------------------------------------------------------- GEMM kernel

@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("layout", [(1, 1), (1, 0), (0, 0)])
@pytest.mark.parametrize("shape", [(200, 256, 96), (128, 128, 64), (64, 384, 1000), (1, 16, 8)])
def test_gemm_kernel_matches_torch(dt, layout, shape):
    """The matrix-core GEMM (every operand layout the inner loop uses,
    ragged M/K tails) against a float64 product of the same values."""
    T = _gpu()
    M, N, K = shape
    a_kc, b_kc = layout
    if not a_kc and M % 8:
        M = 8 * ((M + 7) // 8)
    if (a_kc or b_kc) and K % 8:
        K = 8 * ((K + 7) // 8)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    say(f"case gemm {dt} layout={layout} M={M} N={N} K={K}")
    g = torch.Generator().manual_seed(M * 7 + N * 3 + K)
    A = torch.randn(M, K, generator=g).to(tdt)
    B = torch.randn(N, K, generator=g).to(tdt)
    ref = (A.double() @ B.double().T)
    Ad = (A if a_kc else A.T).contiguous().cuda()
    Bd = (B if b_kc else B.T).contiguous().cuda()
    C = T.diag_gemm(Ad, Bd, M, N, K, bool(a_kc), bool(b_kc))
    torch.cuda.synchronize()
    err = (C.double().cpu() - ref).abs().max().item() / max(ref.abs().max().item(), 1e-30)
    assert err < 1e-5, err


@pytest.fixture
def gemm_core():
    """Select a GEMM core for one test, restore the shape-based choice after."""
    T = _gpu()
    yield T.diag_gemm_core
    T.diag_gemm_core(T.GEMM_CORE_AUTO)


@pytest.mark.parametrize("core", ["auto", "big", "small"])
@pytest.mark.parametrize("shape", [(300, 544, 6160), (257, 3104, 7000), (64, 96, 32), (513, 264, 8),
                                   (1024, 3072, 1000)])
def test_gemm_large_tile_core_matches_torch(gemm_core, core, shape):
    """Both bf16 cores on the k-contiguous layout: the 256x256 core (two
    64-wide direct-to-LDS stages, swizzled rows; the default) and the
    128x128 core (register-staged; forced): ragged M and N tails, a K that
    ends inside a stage, K shorter than one stage."""
    T = _gpu()
    M, N, K = shape
    gemm_core({"big": T.GEMM_CORE_BIG, "small": T.GEMM_CORE_SMALL}.get(core, T.GEMM_CORE_AUTO))
    say(f"case gemm large-tile core={core} M={M} N={N} K={K}")
    g = torch.Generator().manual_seed(M * 5 + N * 11 + K)
    A = torch.randn(M, K, generator=g).to(torch.bfloat16)
    B = torch.randn(N, K, generator=g).to(torch.bfloat16)
    ref = A.double() @ B.double().T
    C = T.diag_gemm(A.cuda(), B.cuda(), M, N, K, True, True)
    torch.cuda.synchronize()
    err = (C.double().cpu() - ref).abs().max().item() / max(ref.abs().max().item(), 1e-30)
    assert err < 1e-5, err


@pytest.mark.parametrize("core", ["auto", "small"])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", [(520, 772, 1000), (3072, 1024, 1024), (16, 8, 8), (1028, 260, 40)])
def test_sgd_epilogue_every_output(gemm_core, core, dt, shape):
    """The fused weight-gradient + SGD product as the inner loop launches it
    (256x256 core by default for bf16, 128x128 core forced or for fp32), on
    several tiles with ragged M, N and K: the fp32 master after
    master -= lr * A B^T against a float64 reference; its bf16 copy equal to
    the master rounded; the transposed current weight round(W0 + master)
    equal, bit for bit, to the rounding of the float sum."""
    T = _gpu()
    if dt == "fp32" and core == "small":
        pytest.skip("fp32 runs the 128x128 core in both modes")
    gemm_core(T.GEMM_CORE_SMALL if core == "small" else T.GEMM_CORE_AUTO)
    M, N, K = shape
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    say(f"case sgd epilogue {dt} core={core} M={M} N={N} K={K}")
    g = torch.Generator().manual_seed(M * 3 + N * 5 + K)
    A = torch.randn(M, K, generator=g).to(tdt)
    B = torch.randn(N, K, generator=g).to(tdt)
    master0 = torch.randn(M, N, generator=g) * 1e-3
    w0 = (torch.randn(M, N, generator=g) * 0.02).to(tdt)
    lr = 0.37
    prod = A.double() @ B.double().T
    ref = master0.double() - lr * prod
    master = master0.cuda()
    copy, cur_t = T.diag_sgd(A.cuda(), B.cuda(), lr, master, w0.cuda())
    torch.cuda.synchronize()
    mc = master.cpu()
    err = (mc.double() - ref).abs().max().item() / (lr * prod).abs().max().item()
    say(f"  master err {err:.2e}")
    assert err < 1e-5
    if dt == "bf16":
        assert torch.equal(copy.cpu(), mc.to(torch.bfloat16))
    assert torch.equal(cur_t.cpu(), (w0.float() + mc).to(tdt).T.contiguous())


@pytest.mark.parametrize("mlp,hd,q", [("swiglu", 128, 2), ("gelu", 64, 3)])
def test_prefill_small_models_large_tile_core(gemm_core, mlp, hd, q):
    """The bf16 small models with every k-contiguous product on the 256x256
    core (its STORE, RESID, GELU and SWIGLU epilogues, W0 + delta, K split
    over workgroups) against the oracle, to the same bar."""
    T = _gpu()
    gemm_core(T.GEMM_CORE_BIG)
    H = 2 if hd <= 64 else 1
    cfg = small_cfg(mlp=mlp, head_dim=hd, n_heads=H, d_model=H * hd, n_fast=q,
                    n_layers=max(3, q + 1))
    r = run_pair(cfg, dtype="bf16", std=0.05, prefill_block=64)
    assert r["loss"] < BAR["bf16"] and r["W"] < BAR["bf16"]
    assert r["loss0"] < BAR["bf16"]
    assert r["dWmax"] < BAR["bf16"] and r["dloss"] < DLOSS_BAR["bf16"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("vocab", [200, 296])
def test_prefill_vocab_not_a_multiple_of_the_tile(dtype, vocab):
    """A vocabulary that ends inside a 256-column tile of the head's
    statistics product (bf16: the 256x256 core, whose tiles also cover
    64-column groups past the vocabulary's end; fp32: the 128x128 core):
    losses and fast weights against the oracle."""
    cfg = small_cfg(vocab=vocab, mlp="swiglu", head_dim=32, n_heads=2, d_model=64)
    r = run_pair(cfg, dtype=dtype, std=0.05, prefill_block=64)
    assert r["loss"] < BAR[dtype] and r["W"] < BAR[dtype]
    assert r["loss0"] < BAR[dtype]
    assert r["dWmax"] < BAR[dtype]
    assert r["dloss"] < DLOSS_BAR[dtype]


# ------------------------------------------------------- whole inner loop

def test_prefill_tiny_fp32_workload():
    """The tiny fp32 workload (2 layers, d 64, hd 16, GELU, window 32, chunk
    16, T 256, lr 0.01): losses and fast weights within 1e-4."""
    r = run_pair(synth.config("c1"))
    assert r["loss"] < BAR["fp32"] and r["W"] < BAR["fp32"]
    assert r["dWmax"] < BAR["fp32"] and r["dloss"] < DLOSS_BAR["fp32"] and r["loss0"] < BAR["fp32"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("mlp,hd,q", [("swiglu", 32, 2), ("gelu", 64, 3), ("swiglu", 16, 3),
                                      ("gelu", 96, 2), ("swiglu", 128, 2)])
def test_prefill_small_models(dtype, mlp, hd, q):
    """Several fast blocks (attention backward through the window, cached
    keys held constant), every head size, both MLPs, a ragged last chunk
    (T = 200 with chunk 32) and several phase-A blocks (block 64)."""
    H = 2 if hd <= 64 else 1
    cfg = small_cfg(mlp=mlp, head_dim=hd, n_heads=H, d_model=H * hd, n_fast=q,
                    n_layers=max(3, q + 1))
    r = run_pair(cfg, dtype=dtype, std=0.05, prefill_block=64)
    assert r["loss"] < BAR[dtype] and r["W"] < BAR[dtype]
    assert r["loss0"] < BAR[dtype]
    assert r["dWmax"] < BAR[dtype]
    assert r["dloss"] < DLOSS_BAR[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("mlp,hd,q", [("swiglu", 32, 2), ("gelu", 64, 1), ("swiglu", 128, 3)])
def test_prefill_static_second_mlp(dtype, mlp, hd, q):
    """The variant whose fast blocks also carry a frozen second MLP after the
    updated one: the gradient into every fast MLP passes through it (for the
    lowest fast block too), several phase-A blocks, a ragged last chunk."""
    H = 2 if hd <= 64 else 1
    cfg = small_cfg(mlp=mlp, head_dim=hd, n_heads=H, d_model=H * hd, n_fast=q,
                    n_layers=max(3, q + 1), static_mlp=1)
    r = run_pair(cfg, dtype=dtype, std=0.05, prefill_block=64)
    assert r["loss"] < BAR[dtype] and r["W"] < BAR[dtype]
    assert r["loss0"] < BAR[dtype]
    assert r["dWmax"] < BAR[dtype]
    assert r["dloss"] < DLOSS_BAR[dtype]


def test_prefill_two_steps_per_chunk_fp32():
    r = run_pair(small_cfg(n_fast=2), steps=2, std=0.05)
    assert r["loss"] < 1e-4 and r["W"] < 1e-4 and r["dWmax"] < 1e-4


def test_window_larger_than_context_and_window_one():
    for W in (1, 1000):
        r = run_pair(small_cfg(window=W, T=96), std=0.05)
        assert r["loss"] < 1e-4 and r["W"] < 1e-4 and r["dWmax"] < 1e-4


def test_chunk_of_one_and_chunk_covering_context():
    for C in (1, 97):
        r = run_pair(small_cfg(T=97), chunk=C, std=0.05, lr0_too=False)
        assert r["loss"] < 1e-4 and r["W"] < 1e-4 and r["dWmax"] < 1e-4


def test_prefill_125m_shape_prefix_bf16():
    """The 125M-shape workload (12 layers, d 768, 12 heads of 64, GELU 3072,
    vocab 32000, window 1024, 3 fast blocks, chunk 256, lr 1e-3) on the first
    1280 tokens: 5 chunks, the window fills, a ragged vocabulary tile."""
    r = run_pair(synth.config("c2"), T=1280)
    assert r["loss"] < BAR["bf16"] and r["W"] < BAR["bf16"]
    assert r["dWmax"] < BAR["bf16"]


def test_prefill_125m_shape_prefix_fp32_check_mode():
    r = run_pair(synth.config("c2"), dtype="fp32", T=768)
    assert r["loss"] < BAR["fp32"] and r["W"] < BAR["fp32"] and r["dWmax"] < BAR["fp32"]


@pytest.mark.parametrize("static", [0, 1])
def test_decode_teacher_forced_matches_oracle(static):
    """Prefill, then greedy decode through two decode-chunk updates; the
    oracle replays the emitted tokens (teacher forcing) and must give the
    same logits and update losses; the argmax must agree wherever the
    oracle's top-2 gap is clear.  static = 1: fast blocks with the frozen
    second MLP."""
    T_ = _gpu()
    cfg = small_cfg(T=64, chunk=16, n_fast=2, window=24, static_mlp=static)
    say(f"case decode small fp32 static_mlp={static}")
    w = [t.float() for t in synth.gen_weights(cfg, std=0.3)]
    x = synth.gen_tokens(cfg, T=64)
    m = T_.Model(cfg, [t.cuda() for t in w], max_chunk=16)
    m.prefill(torch.from_numpy(x).cuda(), 16, 0.05)
    toks, logits, upd = [], [], []
    for i in range(40):
        t, lg, ul = m.decode_step(want_logits=True)
        toks.append(int(t.item()))
        logits.append(lg.cpu().numpy())
        upd.append(float(ul.item()))
    st = O.prefill(cfg, w, x, 16, 0.05, return_state=True)
    first = int(np.argmax(st["last_logits"]))
    assert toks[0] == first
    forced = np.array(toks + [int(np.argmax(logits[-1]))])
    d = O.decode(st, 40, forced=forced)
    L = np.array(logits)
    err = np.abs(L - d["logits"]).max() / np.abs(d["logits"]).max()
    say(f"  decode logits err {err:.2e}")
    assert err < 1e-4
    co = cpp.CppOracle(cfg, w)
    co.prefill(x, 16, 0.05)
    dc = co.decode(41, forced=forced)
    errc = np.abs(L - dc["logits"][:40]).max() / np.abs(dc["logits"]).max()
    say(f"  decode logits err (C++ oracle) {errc:.2e}")
    assert errc < 1e-4
    np.testing.assert_allclose(dc["update_losses"], d["update_losses"], rtol=1e-10)
    for i in range(39):
        srt = np.sort(d["logits"][i])
        if srt[-1] - srt[-2] > 1e-3:
            assert toks[i + 1] == int(np.argmax(d["logits"][i]))
    got = [u for u in upd if not math.isnan(u)]
    assert len(got) == 2 and len(d["update_losses"]) == 2
    np.testing.assert_allclose(got, d["update_losses"], rtol=1e-4)


def _chunk_means(per_pos, T, C):
    """Chunk means of per-position losses (position t predicts t+1)."""
    out = []
    for k in range((T + C - 1) // C):
        seg = per_pos[k * C:min(k * C + C, T - 1)]
        out.append(float(seg.mean()) if len(seg) else 0.0)
    return np.array(out)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("window,block,static", [(48, 256, 0), (48, 64, 0), (1000, 0, 0), (48, 256, 1)])
def test_forward_without_updates_matches_oracle(dtype, window, block, static):
    """The context read with the loaded weights and no update: per-chunk
    losses equal chunk means of the oracle's one-shot forward of the whole
    sequence (no chunking, no cache), and the prefill's losses at lr = 0.
    Block 256 runs the fast blocks over sub-blocks of the frozen-block batch
    (their rings hold window + chunk positions); block 64 spans several
    batches; window 1000 > T is full causal attention."""
    T_ = _gpu()
    cfg = small_cfg(window=window, dtype=dtype, mlp="gelu" if window == 1000 else "swiglu",
                    static_mlp=static)
    say(f"case forward dtype={dtype} window={window} block={block} static_mlp={static}")
    w = synth.gen_weights(cfg, std=0.05)
    if dtype == "fp32":
        w = [t.float() for t in w]
    x = synth.gen_tokens(cfg)
    T, C = cfg["T"], cfg["chunk"]
    m = T_.Model(cfg, [t.cuda() for t in w], max_chunk=C, prefill_block=block)
    tok = torch.from_numpy(x).cuda()
    got = m.forward(tok, C).cpu().numpy()
    ref = _chunk_means(O.sequence_forward_losses(cfg, w, x), T, C)
    e = float(np.max(np.abs(got - ref) / np.abs(ref)))
    p0 = m.prefill(tok, C, 0.0).cpu().numpy()
    e0 = float(np.max(np.abs(got - p0) / np.abs(p0)))
    say(f"  errors: vs oracle {e:.2e}, vs prefill(lr=0) {e0:.2e}")
    assert e < BAR[dtype] and e0 < BAR[dtype]


def test_decode_after_forward_makes_no_update():
    """Greedy decode after the forward-only read: the logits follow the
    oracle's teacher-forced decode at lr = 0 and no update is reported, past
    two decode chunks."""
    T_ = _gpu()
    cfg = small_cfg(T=64, chunk=16, n_fast=2, window=24)
    say("case decode after forward, fp32")
    w = [t.float() for t in synth.gen_weights(cfg, std=0.3)]
    x = synth.gen_tokens(cfg, T=64)
    m = T_.Model(cfg, [t.cuda() for t in w], max_chunk=16)
    m.forward(torch.from_numpy(x).cuda(), 16)
    toks, logits, upd = [], [], []
    for _ in range(40):
        t, lg, ul = m.decode_step(want_logits=True)
        toks.append(int(t.item()))
        logits.append(lg.cpu().numpy())
        upd.append(float(ul.item()))
    st = O.prefill(cfg, w, x, 16, 0.0, return_state=True)
    d = O.decode(st, 40, forced=np.array(toks + [int(np.argmax(logits[-1]))]))
    err = np.abs(np.array(logits) - d["logits"]).max() / np.abs(d["logits"]).max()
    say(f"  decode logits err {err:.2e}")
    assert err < 1e-4
    assert all(math.isnan(u) for u in upd)


def test_prefill_many_contexts_equal_separate_runs():
    """Three independent contexts in one call (their own handles, weights,
    tokens and types; chains interleaved chunk by chunk on their own
    streams): every context's losses and fast weights equal those of its own
    prefill bit for bit, and the first one matches the oracle; decode goes on
    from each; a repeated handle is refused."""
    T_ = _gpu()
    cfgs = [small_cfg(dtype="bf16"), small_cfg(dtype="bf16", weight_seed=222, token_seed=22),
            small_cfg(mlp="gelu", n_fast=1, weight_seed=333, token_seed=33)]
    say("case prefill_many: 3 contexts")
    ws = [synth.gen_weights(c, std=0.05) for c in cfgs]
    ws[2] = [t.float() for t in ws[2]]
    xs = [synth.gen_tokens(c) for c in cfgs]
    ms = [T_.Model(c, [t.cuda() for t in w], max_chunk=32, prefill_block=64) for c, w in zip(cfgs, ws)]
    toks = [torch.from_numpy(x).cuda() for x in xs]
    many = [o.cpu() for o in T_.prefill_many(ms, toks, 32, 0.05)]
    fmany = [[t.cpu() for t in m.fast_weights()] for m in ms]
    nxt = [int(m.decode_step()[0].item()) for m in ms]
    for i, m in enumerate(ms):
        one = m.prefill(toks[i], 32, 0.05).cpu()
        assert torch.equal(one, many[i]), i
        assert all(torch.equal(a, b.cpu()) for a, b in zip(fmany[i], m.fast_weights())), i
        assert 0 <= nxt[i] < cfgs[i]["vocab"]
    ref = O.prefill(cfgs[0], ws[0], xs[0], 32, 0.05)
    e = float(np.max(np.abs(many[0].numpy() - ref["losses"]) / np.abs(ref["losses"])))
    say(f"  context 0 vs oracle: {e:.2e}")
    assert e < BAR["bf16"]
    with pytest.raises(T_.TTTError) as err:
        T_.prefill_many([ms[0], ms[0]], [toks[0], toks[0]], 32, 0.05)
    assert err.value.status == -1


def test_prefill_is_deterministic():
    T_ = _gpu()
    cfg = small_cfg(dtype="bf16")
    say("case determinism")
    w = [t.cuda() for t in synth.gen_weights(cfg, std=0.05)]
    x = torch.from_numpy(synth.gen_tokens(cfg)).cuda()
    m = T_.Model(cfg, w, max_chunk=32)
    a = m.prefill(x, 32, 0.05).cpu()
    fa = [t.cpu() for t in m.fast_weights()]
    b = m.prefill(x, 32, 0.05).cpu()
    fb = [t.cpu() for t in m.fast_weights()]
    assert torch.equal(a, b)
    assert all(torch.equal(p, q) for p, q in zip(fa, fb))


def test_device_detected_errors():
    T_ = _gpu()
    cfg = small_cfg()
    say("case errors")
    w = [t.float().cuda() for t in synth.gen_weights(cfg)]
    m = T_.Model(cfg, w, max_chunk=32)
    bad = torch.from_numpy(synth.gen_tokens(cfg)).cuda()
    bad[17] = cfg["vocab"] + 5
    with pytest.raises(T_.TTTError) as e:
        m.prefill(bad, 32, 0.05)
    assert e.value.status == -4
    ok = torch.from_numpy(synth.gen_tokens(cfg)).cuda()
    with pytest.raises(T_.TTTError) as e:
        m.prefill(ok, 32, 1e30)
    assert e.value.status == -5
    with pytest.raises(T_.TTTError) as e:
        m.prefill(ok, 64, 0.05)        # chunk > max_chunk
    assert e.value.status == -1
    # a context of one position, and a step count of zero, are refused
    # before any work
    with pytest.raises(T_.TTTError) as e:
        m.prefill(ok[:1], 32, 0.05)
    assert e.value.status == -1
    with pytest.raises(T_.TTTError) as e:
        m.forward(ok[:1], 32)
    assert e.value.status == -1
    with pytest.raises(T_.TTTError) as e:
        m.prefill(ok, 32, 0.05, steps=0)
    assert e.value.status == -1
    # decode needs a prefill (or a read without updates) first
    fresh = T_.Model(cfg, w, max_chunk=32)
    with pytest.raises(T_.TTTError) as e:
        fresh.decode_step()
    assert e.value.status == -6
    fresh.close()
    # the model is still usable afterwards
    r = m.prefill(ok, 32, 0.05)
    assert torch.isfinite(r).all()
