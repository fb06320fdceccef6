"""Float64 CPU oracle for the TTT-E2E test-time inner loop.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the package smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP path; the
only common code is the seeded input generator (``synth``), which holds none
of the method's arithmetic.

What it computes (End-to-End Test-Time Training for Long Context):

* the model is a standard decoder-only Transformer whose self-attention is
  sliding-window attention (paper summary page, "Method"; arXiv abstract);
* at test time the model keeps training on the context with plain
  next-token prediction, the loss taken at the end of the network (NVIDIA
  blog, "Our method: compressing context into weights"), one gradient step
  per mini-batch (chunk) of the context (forum post TL;DR, "Inner Loop");
* only MLP layers are updated, attention and embeddings stay static, and
  only the last quarter of the blocks is updated (podcast 6:36 and 7:08);
* optionally (``static_mlp``) each updated block also carries a second,
  frozen MLP that keeps pre-trained knowledge (podcast 7:08); read as a
  pre-LN residual sublayer of the same shape and activation placed after
  the fast MLP, so the gradient into the fast MLP passes through it;
* window ~8K and mini-batch ~1K tokens at the 3B operating point
  (podcast 6:36).

Readings where the pages are silent (each one is also listed in the design
notes of the repository):

* pre-LN blocks, LayerNorm with biased variance, eps 1e-5, no affine
  parameters (gamma = 1, beta = 0) and a final LayerNorm before the head;
* no linear biases; the head ``U`` is untied from the embedding ``E``;
* RoPE on queries and keys, rotate-half pairs ``(i, i + hd/2)`` with
  ``theta_i = base^(-2i/hd)``, absolute positions, angles in float64;
* multi-head attention with scale ``1/sqrt(hd)``; query ``t`` sees keys
  ``j`` with ``t - W < j <= t`` (``W`` keys, itself included);
* GELU uses the exact erf form;
* chunks are cut by input position; position ``t`` predicts ``x[t+1]``; the
  chunk loss is the mean over the chunk's targets; the returned loss of a
  step is measured before that step's update;
* keys and values of earlier chunks are cached as computed when their chunk
  was read (under the fast weights of that time), are never recomputed and
  are constants for the gradient (stop-gradient); with several steps per
  chunk, the chunk is re-read each step and the last read's K/V is kept;
* a chunk without any target (a final chunk of one token) is read and cached
  but makes no update; its loss is reported as 0;
* decoding is greedy (lowest id on ties); the first generated token comes
  from the last prefill chunk's logits; decode positions continue the chunk
  grid from ``T`` and each completed decode chunk makes one update with the
  same loss.

Parity pins (tests/test_oracle_pins.py): finite differences of the fast
weight gradient (also through the frozen second MLP), a zero second MLP
reducing to the plain block, lr = 0 against a one-shot sequence forward, window >= T
against library causal attention, U = 0 and V = 2 closed forms, RoPE shift
invariance, first-order descent, planted-repeat loss drop, decode against
prefill.
"""
from __future__ import annotations

import math
import numpy as np
from scipy.special import erf

__all__ = [
    "OracleModel", "layer_norm", "layer_norm_backward", "rope_cos_sin", "rope_apply",
    "rope_backward", "gelu", "gelu_grad", "silu", "silu_grad", "window_attention",
    "window_attention_backward", "prefill", "decode", "sequence_forward_losses",
    "chunk_loss_and_grad",
]


# --------------------------------------------------------------------------
# Elementary pieces (each is the textbook definition)
# --------------------------------------------------------------------------

def layer_norm(x: np.ndarray, eps: float):
    """LayerNorm over the last axis, biased variance, gamma=1, beta=0.

    Returns ``(y, rstd)`` with ``rstd = 1/sqrt(var + eps)`` (kept for the
    backward pass).
    """
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    return xc * rstd, rstd


def layer_norm_backward(dy: np.ndarray, y: np.ndarray, rstd: np.ndarray) -> np.ndarray:
    """Gradient of ``y = (x - mean) * rstd`` with respect to ``x``.

    ``dx = rstd * (dy - mean(dy) - y * mean(dy * y))`` over the last axis.
    """
    m1 = dy.mean(axis=-1, keepdims=True)
    m2 = (dy * y).mean(axis=-1, keepdims=True)
    return rstd * (dy - m1 - y * m2)


def rope_cos_sin(pos: np.ndarray, head_dim: int, base: float):
    """cos/sin tables ``[n, hd/2]`` for absolute positions, float64 angles."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * i / head_dim)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def rope_apply(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on ``x [n, H, hd]``: pair ``(i, i+hd/2)`` rotated by
    the angle of position ``n`` and frequency ``i``."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_backward(dy: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Transpose of the rotation (rotation by the negative angle)."""
    half = dy.shape[-1] // 2
    d1, d2 = dy[..., :half], dy[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)


def gelu(z):
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def gelu_grad(z):
    cdf = 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return cdf + z * pdf


def silu(z):
    return z / (1.0 + np.exp(-z))


def silu_grad(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def window_attention(q, k, v, qpos, kpos, window: int):
    """Sliding-window causal attention, the plain definition.

    ``q [nq,H,hd]``, ``k, v [nk,H,hd]``; query at position ``t`` attends to
    keys at positions ``j`` with ``t - window < j <= t``.  Returns
    ``(o [nq,H,hd], P [H,nq,nk])``.
    """
    hd = q.shape[-1]
    qpos = np.asarray(qpos)[:, None]
    kpos = np.asarray(kpos)[None, :]
    valid = (kpos <= qpos) & (kpos > qpos - window)
    s = np.matmul(q.transpose(1, 0, 2), k.transpose(1, 2, 0)) / math.sqrt(hd)   # [H,nq,nk]
    s = np.where(valid[None], s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=-1, keepdims=True)
    o = np.matmul(p, v.transpose(1, 0, 2)).transpose(1, 0, 2)                   # [nq,H,hd]
    return o, p


def window_attention_backward(do, q, k, v, p):
    """Gradients of ``o = softmax(q k^T / sqrt(hd)) v`` (masked entries have
    ``p = 0`` and receive no gradient).  Returns ``(dq, dk, dv)``."""
    hd = q.shape[-1]
    scale = 1.0 / math.sqrt(hd)
    doh = do.transpose(1, 0, 2)                                  # [H,nq,hd]
    dv = np.matmul(p.transpose(0, 2, 1), doh).transpose(1, 0, 2)  # [nk,H,hd]
    dp = np.matmul(doh, v.transpose(1, 2, 0))                    # [H,nq,nk]
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    dq = np.matmul(ds, k.transpose(1, 0, 2)).transpose(1, 0, 2) * scale
    dk = np.matmul(ds.transpose(0, 2, 1), q.transpose(1, 0, 2)).transpose(1, 0, 2) * scale
    return dq, dk, dv


def cross_entropy(logits: np.ndarray, targets: np.ndarray):
    """Mean next-token cross-entropy (natural log) and its gradient.

    ``logits [n, V]``; ``targets [m]`` with ``m <= n`` are the targets of the
    first ``m`` rows.  Returns ``(loss, dlogits)``; rows without a target
    get zero gradient.  With ``m = 0`` the loss is 0 and the gradient zero.
    """
    n, V = logits.shape
    m = len(targets)
    dlogits = np.zeros_like(logits)
    if m == 0:
        return 0.0, dlogits
    z = logits[:m]
    zmax = z.max(axis=-1, keepdims=True)
    lse = zmax[:, 0] + np.log(np.exp(z - zmax).sum(axis=-1))
    ll = lse - z[np.arange(m), targets]
    p = np.exp(z - lse[:, None])
    p[np.arange(m), targets] -= 1.0
    dlogits[:m] = p / m
    return float(ll.mean()), dlogits


# --------------------------------------------------------------------------
# Model
# --------------------------------------------------------------------------

class OracleModel:
    """Frozen weights (canonical ``[in, out]`` layout) plus the
    configuration.  Fast weights live in a separate list of dicts, always
    float64.

    ``frozen_dtype``: storage of the frozen matrices.  float64 by default;
    float32 halves the memory of the 3B shape and is exact for weights that
    are bf16 or float32 values.  Every product still runs in float64 (numpy
    promotes the float32 operand exactly), so the arithmetic is the same."""

    def __init__(self, cfg: dict, weights, frozen_dtype=np.float64):
        self.cfg = cfg
        L = cfg["n_layers"]
        names = ["Wq", "Wk", "Wv", "Wo"] + (["W1", "W2"] if cfg["mlp"] == "gelu" else ["Wg", "Wu", "Wd"])
        self.mlp_names = names[4:]
        self.first_fast = L - cfg["n_fast"]
        # the frozen second MLP of the fast blocks (podcast 7:08), when the
        # configuration asks for it: same shapes and activation as the first
        self.static_mlp = bool(cfg.get("static_mlp", 0))
        w = [_to_f64(t) if frozen_dtype == np.float64 else _to_f32_exact(t) for t in weights]
        n_static = cfg["n_fast"] * len(self.mlp_names) if self.static_mlp else 0
        assert len(w) == 2 + L * len(names) + n_static, "weight count does not match the configuration"
        self.E = w[0]
        self.U = w[-1]
        self.layers = []
        self.static = []
        i = 1
        for l in range(L):
            self.layers.append({n: w[i + j] for j, n in enumerate(names)})
            i += len(names)
            if self.static_mlp and l >= self.first_fast:
                self.static.append({n: w[i + j] for j, n in enumerate(self.mlp_names)})
                i += len(self.mlp_names)

    def initial_fast(self):
        """Copies of the MLP matrices of the last ``n_fast`` layers."""
        return [{n: self.layers[l][n].astype(np.float64) for n in self.mlp_names}
                for l in range(self.first_fast, self.cfg["n_layers"])]


def _to_f32_exact(t):
    """float32 copy of a bf16 or float32 tensor (exact: no rounding)."""
    import torch
    if isinstance(t, torch.Tensor):
        assert t.dtype in (torch.bfloat16, torch.float32), "float32 storage needs bf16/float32 weights"
        return t.detach().to("cpu", torch.float32).numpy()
    t = np.asarray(t)
    assert t.dtype == np.float32, "float32 storage needs float32 weights"
    return t


def _to_f64(t):
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def _mlp_forward(cfg, W, b):
    if cfg["mlp"] == "gelu":
        z = b @ W["W1"]
        a = gelu(z)
        return a @ W["W2"], {"z": z, "a": a}
    g = b @ W["Wg"]
    u = b @ W["Wu"]
    a = silu(g) * u
    return a @ W["Wd"], {"g": g, "u": u, "a": a}


def _mlp_backward(cfg, W, b, act, dy, need_input_grad: bool):
    """Returns ``(grads dict, db or None)`` for ``y = mlp(b)``."""
    if cfg["mlp"] == "gelu":
        grads = {"W2": act["a"].T @ dy}
        da = dy @ W["W2"].T
        dz = da * gelu_grad(act["z"])
        grads["W1"] = b.T @ dz
        db = dz @ W["W1"].T if need_input_grad else None
        return grads, db
    grads = {"Wd": act["a"].T @ dy}
    da = dy @ W["Wd"].T
    g, u = act["g"], act["u"]
    dg = da * u * silu_grad(g)
    du = da * silu(g)
    grads["Wg"] = b.T @ dg
    grads["Wu"] = b.T @ du
    db = (dg @ W["Wg"].T + du @ W["Wu"].T) if need_input_grad else None
    return grads, db


def _heads(x, cfg):
    return x.reshape(x.shape[0], cfg["n_heads"], cfg["head_dim"])


def forward_chunk(model: OracleModel, fast, cache, tokens, pos0: int):
    """Forward ``tokens`` at positions ``pos0 ..`` through all layers.

    ``cache[l]`` holds ``(pos, k, v)`` of earlier positions (read only).
    Returns the saved activations and the logits.
    """
    cfg = model.cfg
    eps, W = cfg["ln_eps"], cfg["window"]
    n = len(tokens)
    pos = np.arange(pos0, pos0 + n)
    cos, sin = rope_cos_sin(pos, cfg["head_dim"], cfg["rope_base"])
    h = model.E[np.asarray(tokens)].astype(np.float64)
    acts = []
    for l in range(cfg["n_layers"]):
        Wl = model.layers[l]
        fl = l - model.first_fast
        Wm = fast[fl] if fl >= 0 else Wl
        a, r1 = layer_norm(h, eps)
        q = rope_apply(_heads(a @ Wl["Wq"], cfg), cos, sin)
        k = rope_apply(_heads(a @ Wl["Wk"], cfg), cos, sin)
        v = _heads(a @ Wl["Wv"], cfg)
        cpos, ck, cv = cache[l]
        kall = np.concatenate([ck, k], axis=0)
        vall = np.concatenate([cv, v], axis=0)
        kpos = np.concatenate([cpos, pos])
        o, p = window_attention(q, kall, vall, pos, kpos, W)
        h2 = h + o.reshape(n, -1) @ Wl["Wo"]
        b, r2 = layer_norm(h2, eps)
        m, mact = _mlp_forward(cfg, Wm, b)
        # saved for the cache (every layer) and for the backward pass (the
        # MLP of every fast block; the attention of fast blocks above the
        # first), nothing else
        A = dict(k=k, v=v)
        if fl >= 0:
            A.update(b=b, r2=r2, mact=mact)
        if fl > 0:
            # the attention probabilities are not kept: the backward pass
            # recomputes them from the same inputs (identical values)
            A.update(h=h, a=a, r1=r1, q=q, kall=kall, vall=vall, kpos=kpos, ncache=len(cpos), h2=h2)
        del p, kall, vall
        h = h2 + m
        if fl >= 0 and model.static_mlp:
            # frozen second MLP after the fast one, its own pre-LayerNorm
            c, r3 = layer_norm(h, eps)
            m2, mact2 = _mlp_forward(cfg, model.static[fl], c)
            A.update(c=c, r3=r3, mact2=mact2)
            h = h + m2
        acts.append(A)
    f, rf = layer_norm(h, eps)
    logits = f @ model.U
    return dict(layers=acts, hL=h, f=f, rf=rf, logits=logits, pos=pos, cos=cos, sin=sin)


def backward_chunk(model: OracleModel, fast, fw, dlogits):
    """Gradient of the chunk loss with respect to the fast weights only.

    The backward stops at the first fast MLP; cached keys and values are
    constants.  Returns a list (per fast layer) of gradient dicts.
    """
    cfg = model.cfg
    L = cfg["n_layers"]
    df = dlogits @ model.U.T
    dh = layer_norm_backward(df, fw["f"], fw["rf"])
    grads = [None] * cfg["n_fast"]
    for l in range(L - 1, model.first_fast - 1, -1):
        A = fw["layers"][l]
        Wl = model.layers[l]
        fl = l - model.first_fast
        need = l > model.first_fast
        if model.static_mlp:
            # through the frozen second MLP (its weight gradient is not used)
            _, dc = _mlp_backward(cfg, model.static[fl], A["c"], A["mact2"], dh, True)
            dh = dh + layer_norm_backward(dc, A["c"], A["r3"])
        g, db = _mlp_backward(cfg, fast[fl], A["b"], A["mact"], dh, need)
        grads[fl] = g
        if not need:
            break
        dh2 = dh + layer_norm_backward(db, A["b"], A["r2"])
        n = dh2.shape[0]
        do = _heads(dh2 @ Wl["Wo"].T, cfg)
        _, p = window_attention(A["q"], A["kall"], A["vall"], fw["pos"], A["kpos"], cfg["window"])
        dq, dkall, dvall = window_attention_backward(do, A["q"], A["kall"], A["vall"], p)
        del p
        nc = A["ncache"]
        dk = dkall[nc:]                      # cached keys/values: stop-gradient
        dv = dvall[nc:]
        dq = rope_backward(dq, fw["cos"], fw["sin"])
        dk = rope_backward(dk, fw["cos"], fw["sin"])
        da = (dq.reshape(n, -1) @ Wl["Wq"].T + dk.reshape(n, -1) @ Wl["Wk"].T
              + dv.reshape(n, -1) @ Wl["Wv"].T)
        dh = dh2 + layer_norm_backward(da, A["a"], A["r1"])
    return grads


def empty_cache(cfg):
    H, hd = cfg["n_heads"], cfg["head_dim"]
    return [(np.zeros(0, dtype=np.int64), np.zeros((0, H, hd)), np.zeros((0, H, hd)))
            for _ in range(cfg["n_layers"])]


def _commit(cfg, cache, fw, keep: int):
    """Append the chunk's keys/values to every layer's cache, keeping the
    newest ``keep`` positions."""
    out = []
    for l, (cpos, ck, cv) in enumerate(cache):
        A = fw["layers"][l]
        npos = np.concatenate([cpos, fw["pos"]])
        nk = np.concatenate([ck, A["k"]], axis=0)
        nv = np.concatenate([cv, A["v"]], axis=0)
        out.append((npos[-keep:], nk[-keep:], nv[-keep:]))
    return out


def chunk_loss_and_grad(model, fast, cache, tokens, targets, pos0):
    """Loss of one chunk (mean CE over its targets) and the fast-weight
    gradient, without changing anything.  Used by the finite-difference
    pin."""
    fw = forward_chunk(model, fast, cache, tokens, pos0)
    loss, dl = cross_entropy(fw["logits"], np.asarray(targets))
    return loss, backward_chunk(model, fast, fw, dl), fw


def _sgd(fast, grads, lr):
    for f, g in zip(fast, grads):
        for n in f:
            f[n] = f[n] - lr * g[n]


def prefill(cfg, weights, tokens, chunk: int, lr: float, steps: int = 1, pos_offset: int = 0,
            model: OracleModel | None = None, return_state: bool = False, max_chunks=None,
            progress: bool = False):
    """The inner loop over a whole context.

    For each chunk ``k`` (positions ``[kC, min(kC+C, T))``) and each step:
    forward with the current fast weights, attention over cached keys of
    earlier chunks plus causal in-chunk keys; mean next-token CE over the
    chunk's targets; gradient into the fast MLP weights only; SGD
    ``phi <- phi - lr * g``.  Then the chunk's K/V (last read) join the cache.

    Returns ``dict(losses [N*steps], fast, last_logits, ...)``.
    ``max_chunks`` stops early (bounded CPU-baseline samples); ``progress``
    prints a line per chunk.
    """
    model = model or OracleModel(cfg, weights)
    tokens = np.asarray(tokens)
    T = len(tokens)
    C = int(chunk)
    fast = model.initial_fast()
    cache = empty_cache(cfg)
    keep = cfg["window"] + C
    losses = []
    last_logits = None
    nchunks = (T + C - 1) // C
    if max_chunks is not None:
        nchunks = min(nchunks, max_chunks)
    for k in range(nchunks):
        p0, p1 = k * C, min(k * C + C, T)
        toks = tokens[p0:p1]
        tgt = tokens[p0 + 1:min(p1 + 1, T)]
        for s in range(steps):
            fw = forward_chunk(model, fast, cache, toks, p0 + pos_offset)
            loss, dl = cross_entropy(fw["logits"], tgt)
            losses.append(loss)
            if len(tgt) > 0:
                grads = backward_chunk(model, fast, fw, dl)
                _sgd(fast, grads, lr)
        cache = _commit(cfg, cache, fw, keep)
        last_logits = fw["logits"][-1].copy()
        if progress:
            print(f"  oracle chunk {k + 1}/{nchunks}: loss {losses[-steps]:.6f}", flush=True)
    out = dict(losses=np.array(losses), fast=fast, last_logits=last_logits)
    if return_state:
        out.update(model=model, cache=cache, T=T, pos_offset=pos_offset, chunk=C, lr=lr,
                   steps=steps)
    return out


def decode(state: dict, n_tokens: int, forced=None):
    """Greedy decode after ``prefill(..., return_state=True)``.

    Position ``p >= T`` is read with the current fast weights and its K/V
    join the cache; the next token is ``argmax`` of its logits (lowest id on
    ties) unless ``forced`` gives it (teacher forcing).  When the decode
    positions ``[T + mC, T + (m+1)C)`` are complete, that chunk makes the
    same update as a prefill chunk (its ``C`` targets are the tokens that
    followed each position).

    Returns ``dict(tokens [n], logits [n, V], update_losses list)``; the
    state's fast weights and cache are updated in place.
    """
    model = state["model"]
    cfg = model.cfg
    C, lr, steps = state["chunk"], state["lr"], state["steps"]
    fast, cache = state["fast"], state["cache"]
    keep = cfg["window"] + C
    T, off = state["T"], state["pos_offset"]
    nxt = int(np.argmax(state["last_logits"])) if forced is None else int(forced[0])
    toks, logits_all, upd = [], [], []
    chunk_toks = []
    for i in range(n_tokens):
        p = T + i
        tok = nxt
        toks.append(tok)
        chunk_toks.append(tok)
        fw = forward_chunk(model, fast, cache, [tok], p + off)
        cache = _commit(cfg, cache, fw, keep)
        lg = fw["logits"][0]
        logits_all.append(lg.copy())
        if forced is not None and i + 1 < len(forced):
            nxt = int(forced[i + 1])
        else:
            nxt = int(np.argmax(lg))
        if (i + 1) % C == 0:
            c0 = p + 1 - C
            tgt = np.array(chunk_toks[1:] + [nxt])
            before = [(cp[cp < c0 + off], ck[cp < c0 + off], cv[cp < c0 + off])
                      for cp, ck, cv in cache]
            for s in range(steps):
                fwc = forward_chunk(model, fast, before, np.array(chunk_toks), c0 + off)
                loss, dl = cross_entropy(fwc["logits"], tgt)
                upd.append(loss)
                _sgd(fast, backward_chunk(model, fast, fwc, dl), lr)
            # as in prefill, the chunk's K/V from its last read are the ones kept
            cache = _commit(cfg, before, fwc, keep)
            chunk_toks = []
    state["cache"] = cache
    state["T"] = T + n_tokens
    state["last_logits"] = None
    return dict(tokens=np.array(toks), logits=np.array(logits_all), update_losses=upd)


def sequence_forward_losses(cfg, weights, tokens, pos_offset: int = 0, frozen_dtype=np.float64):
    """One-shot forward of the whole sequence with the initial weights (no
    chunks, no cache, no updates); per-position next-token losses
    ``[T-1]``."""
    model = OracleModel(cfg, weights, frozen_dtype=frozen_dtype)
    tokens = np.asarray(tokens)
    fw = forward_chunk(model, model.initial_fast(), empty_cache(cfg), tokens, pos_offset)
    z = fw["logits"][:-1]
    zmax = z.max(axis=-1, keepdims=True)
    lse = zmax[:, 0] + np.log(np.exp(z - zmax).sum(axis=-1))
    return lse - z[np.arange(len(tokens) - 1), tokens[1:]]


def fast_weights_canonical(out: dict):
    """Flatten the final fast weights to a list in canonical order
    (per fast layer, MLP matrices in ``[in, out]`` layout)."""
    res = []
    for f in out["fast"]:
        res.extend(f[n] for n in f)
    return res
