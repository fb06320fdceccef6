"""Seeded synthetic workloads for the TTT-E2E test-time inner loop.

The pages on End-to-End Test-Time Training for Long Context evaluate on
long natural-language contexts with trained 3B models; neither the data nor
the weights are available, so every workload here is synthetic:

* tokens: i.i.d. Zipf(1.1) over the vocabulary (rank r has probability
  proportional to r^-1.1, token id = r - 1), then segments of ``seg`` tokens
  are copied from ``D`` positions back, with ``D`` drawn uniformly from
  ``[dmin, min(dmax, s)]`` and ``dmin`` larger than the attention window, so
  a copy can only be predicted through the long-range channel (the weight
  updates), never through sliding-window attention;
* weights: every matrix i.i.d. N(0, 0.02^2) from a per-tensor seed, rounded
  to bfloat16 (round to nearest even) for bf16 configurations before any
  consumer sees them.

Canonical weight layout (shared by the C-ABI and the oracle): every
projection is stored ``[in, out]`` row-major, so a layer computes
``y = x @ W``.  Order: ``E [V,d]``; per layer ``Wq, Wk, Wv, Wo [d,d]`` then
either ``W1 [d,F], W2 [F,d]`` (GELU) or ``Wg [d,F], Wu [d,F], Wd [F,d]``
(SwiGLU); last ``U [d,V]`` (head, untied from ``E``).
"""
from __future__ import annotations

import copy
import numpy as np

# Model shapes and inner-loop settings of the five workloads.  Window 8192 and
# mini-batch 1024 follow the podcast page (6:36, "window of 8,000 tokens",
# "mini-batches of 1,000 tokens"); the last-quarter rule for the fast layers
# follows the same page (7:08).
CONFIGS = {
    "c1": dict(name="tiny-fp32", n_layers=2, d_model=64, n_heads=4, head_dim=16,
               d_ff=256, vocab=256, window=32, n_fast=1, mlp="gelu", dtype="fp32",
               T=256, chunk=16, lr=0.01, steps=1,
               seg=16, period=64, dmin=33, dmax=None, token_seed=1, weight_seed=101),
    "c2": dict(name="125M-shape", n_layers=12, d_model=768, n_heads=12, head_dim=64,
               d_ff=3072, vocab=32000, window=1024, n_fast=3, mlp="gelu", dtype="bf16",
               T=8192, chunk=256, lr=1e-3, steps=1,
               seg=64, period=256, dmin=2048, dmax=8192, token_seed=2, weight_seed=102),
    # lr is not given for this workload; 3e-4 is the log-midpoint of the
    # neighbouring workloads' 1e-3 (125M) and 1e-4 (3B).
    "c3": dict(name="760M-shape", n_layers=24, d_model=1536, n_heads=16, head_dim=96,
               d_ff=4096, vocab=32000, window=4096, n_fast=6, mlp="swiglu", dtype="bf16",
               T=32768, chunk=512, lr=3e-4, steps=1,
               seg=128, period=512, dmin=8192, dmax=32768, token_seed=3, weight_seed=103),
    "c4": dict(name="3B-shape-128K", n_layers=28, d_model=3072, n_heads=24, head_dim=128,
               d_ff=8192, vocab=32000, window=8192, n_fast=7, mlp="swiglu", dtype="bf16",
               T=131072, chunk=1024, lr=1e-4, steps=1,
               seg=256, period=1024, dmin=16384, dmax=65536, token_seed=4, weight_seed=104),
    "c5": dict(name="3B-shape-512K-decode", n_layers=28, d_model=3072, n_heads=24, head_dim=128,
               d_ff=8192, vocab=32000, window=8192, n_fast=7, mlp="swiglu", dtype="bf16",
               T=524288, chunk=1024, lr=1e-4, steps=1, decode_tokens=512,
               seg=256, period=1024, dmin=16384, dmax=65536, token_seed=5, weight_seed=104),
}


def config(name_or_cfg, **overrides) -> dict:
    """Return a copy of a named workload (or of a dict) with overrides."""
    base = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    cfg = copy.deepcopy(base)
    cfg.update(overrides)
    cfg.setdefault("rope_base", 10000.0)
    cfg.setdefault("ln_eps", 1e-5)
    assert cfg["n_heads"] * cfg["head_dim"] == cfg["d_model"], "d_model = heads * head_dim"
    assert cfg["mlp"] in ("gelu", "swiglu")
    assert cfg["dtype"] in ("fp32", "bf16")
    assert 1 <= cfg["n_fast"] <= cfg["n_layers"]
    return cfg


def _zipf_cdf(vocab: int, s: float) -> np.ndarray:
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    p = ranks ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


def gen_tokens(cfg: dict, T: int | None = None, seed: int | None = None,
               zipf_s: float = 1.1, plant: bool = True, return_copies: bool = False):
    """Zipf(1.1) token stream with planted long-range copies.

    Copies are placed at slots ``s = dmin, dmin+period, ...`` while
    ``s + seg <= T``; each copies ``x[s-D : s-D+seg]`` to ``x[s : s+seg]``
    with ``D ~ U{dmin .. min(dmax, s)}``, in increasing ``s`` (so a source may
    itself be a copy).  Returns int32 ``[T]`` (and a bool mask of copied
    positions when ``return_copies``).
    """
    T = cfg["T"] if T is None else int(T)
    seed = cfg["token_seed"] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    cdf = _zipf_cdf(cfg["vocab"], zipf_s)
    u = rng.random(T)
    x = np.searchsorted(cdf, u, side="right").astype(np.int64)
    x = np.minimum(x, cfg["vocab"] - 1).astype(np.int32)
    copied = np.zeros(T, dtype=bool)
    if plant:
        seg, period, dmin = cfg["seg"], cfg["period"], cfg["dmin"]
        dmax = cfg["dmax"] if cfg.get("dmax") is not None else T
        s = dmin
        while s + seg <= T:
            hi = min(dmax, s)
            D = int(rng.integers(dmin, hi + 1))
            x[s:s + seg] = x[s - D:s - D + seg].copy()
            copied[s:s + seg] = True
            s += period
    return (x, copied) if return_copies else x


def _has_static(cfg: dict, l: int) -> bool:
    """Layer l carries the frozen second MLP (fast layers of a static_mlp
    variant)."""
    return bool(cfg.get("static_mlp", 0)) and l >= cfg["n_layers"] - cfg["n_fast"]


def weight_names(cfg: dict) -> list[str]:
    names = ["E"]
    mlp = ["W1", "W2"] if cfg["mlp"] == "gelu" else ["Wg", "Wu", "Wd"]
    smlp = ["S1", "S2"] if cfg["mlp"] == "gelu" else ["Sg", "Su", "Sd"]
    for l in range(cfg["n_layers"]):
        names += [f"L{l}.{n}" for n in ["Wq", "Wk", "Wv", "Wo"] + mlp]
        if _has_static(cfg, l):
            names += [f"L{l}.{n}" for n in smlp]
    names.append("U")
    return names


def weight_shapes(cfg: dict) -> list[tuple[int, int]]:
    d, F, V = cfg["d_model"], cfg["d_ff"], cfg["vocab"]
    shapes = [(V, d)]
    mlp = [(d, F), (F, d)] if cfg["mlp"] == "gelu" else [(d, F), (d, F), (F, d)]
    for l in range(cfg["n_layers"]):
        shapes += [(d, d)] * 4 + mlp
        if _has_static(cfg, l):
            shapes += mlp
    shapes.append((d, V))
    return shapes


def n_weights(cfg: dict) -> int:
    return len(weight_shapes(cfg))


def gen_weights(cfg: dict, seed: int | None = None, device="cpu", std: float = 0.02,
                storage_dtype=None):
    """List of torch tensors, canonical order and layout, i.i.d. N(0, std^2).

    Tensor ``i`` is drawn from its own generator seeded with
    ``seed * 1_000_003 + i`` on ``device``, so tensors are independent of
    each other's sizes.  bf16 configurations round to bfloat16; fp32 ones keep
    float32.  ``storage_dtype`` forces a torch dtype (e.g. float32 holding
    bf16-rounded values for the fp32 check mode of a bf16 workload).
    """
    import torch

    seed = cfg["weight_seed"] if seed is None else seed
    out = []
    for i, shp in enumerate(weight_shapes(cfg)):
        g = torch.Generator(device=device)
        g.manual_seed(int(seed) * 1_000_003 + i)
        w = torch.randn(shp, generator=g, device=device, dtype=torch.float32) * std
        if cfg["dtype"] == "bf16":
            w = w.to(torch.bfloat16)
        if storage_dtype is not None:
            w = w.to(storage_dtype)
        out.append(w.contiguous())
    return out
