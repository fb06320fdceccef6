"""Stored float64-oracle results for the parity tests of the larger workloads.

The oracle needs minutes to an hour on the host for these contexts, far too
long inside a GPU test, so its results are computed once by running this
file and stored next to it (``<case>.npz``).  The script calls only the
oracle (``oracle/``) and the seeded input generator (``synth/``): no stored
value comes from the HIP path.

    python tests/golden/oracle_fixtures.py c2_full c3_5120 c3_full c4_10240 c4_20480

Each case is a workload read with the test-time inner loop over a prefix of
its context (every chunk's loss returned before that chunk's update, End-to-
End Test-Time Training for Long Context, forum post TL;DR "Inner Loop"):

* ``c2_full``   the 125M-shape workload over its whole context (8192 tokens,
  32 chunks of 256, window 1024);
* ``c3_5120``   the 760M-shape workload (head size 96, SwiGLU, 6 fast blocks)
  over 5120 tokens: the 4096-key window fills and the fast blocks' K/V rings
  (4096 + 512 positions) wrap;
* ``c3_full``   the same workload over its whole context (32768 tokens, 64
  chunks of 512);
* ``c4_10240``  the 3B-shape workload over 10240 tokens: full 8192-key
  windows, the fast blocks' rings (8192 + 1024 positions) wrap, two blocks
  of the frozen layers;
* ``c4_20480``  the same over 20480 tokens: 20 chunks, three blocks of the
  frozen layers, the fast rings wrapped twice.

Stored per case: every chunk loss; for every fast matrix (canonical
``[in][out]`` layout) its change over the whole prefill, dW = W - W0, at one
element of every 64 x 64 tile (the element chosen by ``sample_indices``), the
largest |dW| and ||dW||_F over the whole matrix; the logits of the last
position; and fingerprints of the weights and tokens, so that a test can tell
whether its host generated the same inputs.
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

CASES = {
    "c2_full": dict(workload="c2", T=8192),
    "c3_5120": dict(workload="c3", T=5120),
    "c3_full": dict(workload="c3", T=32768),
    "c4_10240": dict(workload="c4", T=10240),
    "c4_20480": dict(workload="c4", T=20480),
}
# The positions of the 512K-context workload on the tiny fp32 model: its
# chunk of 1024, a window of 32, 525312 = 513 x 1024 tokens (positions up
# to 2^19 + 1023).  Stored: every chunk loss, the fast weights after the
# prefill (float64, whole) and the keys/values of the last `window`
# positions of every layer (all that later decode positions can attend to),
# so that a test can continue with the oracle's decode from that state.
LONG = {"c1_525k": dict(workload="c1", T=525312, chunk=1024, window=32)}
SAMPLE_BLOCK = 64


def case_config(case: str) -> dict:
    if case in LONG:
        c = LONG[case]
        return synth.config(c["workload"], T=c["T"], chunk=c["chunk"], window=c["window"])
    c = CASES[case]
    return synth.config(c["workload"], T=c["T"])


def path(case: str) -> str:
    return os.path.join(HERE, case + ".npz")


def sample_indices(shape, block: int = SAMPLE_BLOCK, seed: int = 0) -> np.ndarray:
    """Flat indices of one element in every ``block x block`` tile of a
    ``[R][C]`` matrix (ragged edge tiles included), chosen by a seeded
    generator: every tile of every GPU launch holds several samples."""
    R, C = shape
    rng = np.random.Generator(np.random.PCG64(seed + 7919 * R + C))
    r0 = np.arange(0, R, block)
    c0 = np.arange(0, C, block)
    rh = np.minimum(block, R - r0)
    ch = np.minimum(block, C - c0)
    rr = r0[:, None] + (rng.random((len(r0), len(c0))) * rh[:, None]).astype(np.int64)
    cc = c0[None, :] + (rng.random((len(r0), len(c0))) * ch[None, :]).astype(np.int64)
    return (rr * C + cc).ravel()


def fingerprint(tensors) -> str:
    """blake2b over the bytes of every tensor in order (torch or numpy)."""
    h = hashlib.blake2b(digest_size=16)
    for t in tensors:
        try:
            import torch
            if isinstance(t, torch.Tensor):
                t = t.detach().cpu().contiguous().view(torch.uint8).numpy()
        except ImportError:  # pragma: no cover
            pass
        h.update(np.ascontiguousarray(t).tobytes())
    return h.hexdigest()


def compute(case: str) -> str:
    from oracle import ttt_oracle as O
    cfg = case_config(case)
    T, C, lr = cfg["T"], cfg["chunk"], cfg["lr"]
    t0 = time.time()
    w = synth.gen_weights(cfg)
    x = synth.gen_tokens(cfg)
    wfp, xfp = fingerprint(w), fingerprint([x])
    print(f"{case}: inputs generated in {time.time() - t0:.0f} s (weights {wfp}, tokens {xfp})", flush=True)
    model = O.OracleModel(cfg, w, frozen_dtype=np.float32)
    del w
    t0 = time.time()
    out = O.prefill(cfg, None, x, C, lr, model=model, progress=True)
    print(f"{case}: oracle prefill of {T} tokens in {time.time() - t0:.0f} s", flush=True)
    res = dict(losses=out["losses"], last_logits=out["last_logits"].astype(np.float32), T=T, chunk=C, lr=lr,
               weights_fingerprint=wfp, tokens_fingerprint=xfp, workload=CASES[case]["workload"])
    names = model.mlp_names
    i = 0
    for j, f in enumerate(out["fast"]):
        l = model.first_fast + j
        for n in names:
            dw = f[n] - model.layers[l][n]          # float64 - exact float32 W0
            res[f"dW_sample_{i}"] = dw.ravel()[sample_indices(dw.shape)].astype(np.float32)
            res[f"dW_absmax_{i}"] = float(np.abs(dw).max())
            res[f"dW_fro_{i}"] = float(np.linalg.norm(dw))
            res[f"shape_{i}"] = np.array(dw.shape)
            i += 1
    res["n_mats"] = i
    np.savez_compressed(path(case), **res)
    return path(case)


def compute_long(case: str) -> str:
    from oracle import ttt_oracle as O
    cfg = case_config(case)
    T, C, lr, W = cfg["T"], cfg["chunk"], cfg["lr"], cfg["window"]
    w = synth.gen_weights(cfg)
    x = synth.gen_tokens(cfg)
    t0 = time.time()
    st = O.prefill(cfg, w, x, C, lr, return_state=True)
    print(f"{case}: oracle prefill of {T} tokens in {time.time() - t0:.0f} s", flush=True)
    res = dict(losses=st["losses"], last_logits=st["last_logits"], T=T, chunk=C, lr=lr, window=W,
               weights_fingerprint=fingerprint(w), tokens_fingerprint=fingerprint([x]),
               workload=LONG[case]["workload"])
    for j, f in enumerate(st["fast"]):
        for n, a in f.items():
            res[f"fast_{j}_{n}"] = a
    for l, (cp, ck, cv) in enumerate(st["cache"]):
        keep = cp >= T - W
        res[f"cache_pos_{l}"], res[f"cache_k_{l}"], res[f"cache_v_{l}"] = cp[keep], ck[keep], cv[keep]
    np.savez_compressed(path(case), **res)
    return path(case)


def load_long_state(case: str, weights):
    """The oracle's state after the stored prefill, ready for oracle.decode."""
    from oracle import ttt_oracle as O
    fx = np.load(path(case))
    cfg = case_config(case)
    model = O.OracleModel(cfg, weights)
    names = model.mlp_names
    fast = [{n: fx[f"fast_{j}_{n}"].copy() for n in names} for j in range(cfg["n_fast"])]
    cache = [(fx[f"cache_pos_{l}"], fx[f"cache_k_{l}"], fx[f"cache_v_{l}"]) for l in range(cfg["n_layers"])]
    return dict(model=model, fast=fast, cache=cache, T=int(fx["T"]), pos_offset=0, chunk=int(fx["chunk"]),
                lr=float(fx["lr"]), steps=1, last_logits=fx["last_logits"].copy())


if __name__ == "__main__":
    for c in sys.argv[1:] or list(CASES) + list(LONG):
        print("wrote", compute_long(c) if c in LONG else compute(c), flush=True)
