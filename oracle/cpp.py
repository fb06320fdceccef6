"""ctypes binding of the plain C++ float64 oracle (``ttt_oracle.cpp``).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
package smoke check and the benchmark's CPU-baseline leg may load it.  This
module only marshals arguments; the computation is in the C++ source.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# TTT_ORACLE_LIB points the binding at another build of the same source (a
# mutated copy, when checking that the pins catch a planted mistake).
LIB_PATH = os.environ.get("TTT_ORACLE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "libttt_oracle.so")


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "d_model", "n_heads", "head_dim", "d_ff",
                                              "vocab", "window", "n_fast", "swiglu", "static_mlp")] + \
               [("rope_base", ctypes.c_double), ("ln_eps", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            # the checker is built on first use if the build step has not run
            import importlib.util
            spec = importlib.util.spec_from_file_location(
                "_ttt_oracle_build", os.path.join(os.path.dirname(os.path.abspath(__file__)), "build.py"))
            b = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(b)
            b.build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, dp = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        sig = {
            "orc_n_weights": ([ctypes.POINTER(_Cfg)], ctypes.c_int),
            "orc_model_new": ([ctypes.POINTER(_Cfg), ctypes.POINTER(vp)], vp),
            "orc_model_free": ([vp], None),
            "orc_prefill": ([vp, vp, i64, i32, dp, i32, i64, vp, vp], ctypes.c_int),
            "orc_decode": ([vp, i32, vp, vp, vp, vp, ctypes.POINTER(i32)], ctypes.c_int),
            "orc_fast_weight": ([vp, i32, i32, vp], ctypes.c_int),
            "orc_set_fast_weight": ([vp, i32, i32, vp], ctypes.c_int),
            "orc_chunk_loss_grad": ([vp, vp, i32, vp, i32, i64, vp], dp),
            "orc_read": ([vp, vp, i32, i64, i32], ctypes.c_int),
            "orc_rope": ([vp, i32, i32, i32, vp, dp, i32], None),
            "orc_layer_norm": ([vp, i32, i32, dp, vp], None),
            "orc_attention": ([vp, vp, vp, i32, i32, i32, i32, vp, vp, i64, vp], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _f64(t) -> np.ndarray:
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return np.ascontiguousarray(t.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(t, dtype=np.float64))


class CppOracle:
    """One model (frozen weights, fast weights, K/V cache) of the C++ oracle."""

    def __init__(self, cfg: dict, weights):
        self.cfg = cfg
        self.c = _Cfg(cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["head_dim"], cfg["d_ff"],
                      cfg["vocab"], cfg["window"], cfg["n_fast"], int(cfg["mlp"] == "swiglu"),
                      int(cfg.get("static_mlp", 0)), float(cfg.get("rope_base", 10000.0)),
                      float(cfg.get("ln_eps", 1e-5)))
        n = lib().orc_n_weights(ctypes.byref(self.c))
        assert len(weights) == n, f"{len(weights)} weights given, the configuration takes {n}"
        ws = [_f64(w) for w in weights]
        arr = (ctypes.c_void_p * n)(*[w.ctypes.data for w in ws])
        self.h = lib().orc_model_new(ctypes.byref(self.c), arr)
        self.n_mlp = 3 if cfg["mlp"] == "swiglu" else 2
        d, F = cfg["d_model"], cfg["d_ff"]
        self.shapes = [(d, F), (F, d)] if self.n_mlp == 2 else [(d, F), (d, F), (F, d)]

    def __del__(self):
        if getattr(self, "h", None):
            lib().orc_model_free(self.h)
            self.h = None

    def prefill(self, tokens, chunk: int, lr: float, steps: int = 1, pos_offset: int = 0):
        x = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        T = len(x)
        nch = (T + chunk - 1) // chunk
        losses = np.zeros(nch * steps)
        last = np.zeros(self.cfg["vocab"])
        rc = lib().orc_prefill(self.h, _ptr(x), T, chunk, float(lr), steps, pos_offset, _ptr(losses),
                               _ptr(last))
        assert rc == 0, rc
        return dict(losses=losses, last_logits=last, fast=self.fast_weights())

    def decode(self, n: int, forced=None):
        f = None if forced is None else np.ascontiguousarray(np.asarray(forced, dtype=np.int32))
        assert f is None or len(f) == n
        toks = np.zeros(n, dtype=np.int32)
        logits = np.zeros((n, self.cfg["vocab"]))
        upd = np.zeros(max(1, n * 4))
        nu = ctypes.c_int32(0)
        rc = lib().orc_decode(self.h, n, None if f is None else _ptr(f), _ptr(toks), _ptr(logits),
                              _ptr(upd), ctypes.byref(nu))
        assert rc == 0, rc
        return dict(tokens=toks, logits=logits, update_losses=upd[:nu.value].tolist())

    def fast_weights(self):
        """Fast matrices in canonical order (per fast layer, MLP order), [in][out]."""
        out = []
        for f in range(self.cfg["n_fast"]):
            for j, shp in enumerate(self.shapes):
                a = np.zeros(shp)
                assert lib().orc_fast_weight(self.h, f, j, _ptr(a)) == 0
                out.append(a)
        return out

    def set_fast_weight(self, f: int, j: int, a):
        a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
        assert a.shape == self.shapes[j]
        assert lib().orc_set_fast_weight(self.h, f, j, _ptr(a)) == 0

    def read(self, tokens, pos0: int, keep_extra: int):
        """Read tokens into the cache without an update (keeps window + keep_extra positions)."""
        x = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        assert lib().orc_read(self.h, _ptr(x), len(x), pos0, keep_extra) == 0

    def chunk_loss_grad(self, tokens, targets, pos0: int, grads: bool = True):
        x = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        t = np.ascontiguousarray(np.asarray(targets, dtype=np.int32))
        size = sum(a * b for a, b in self.shapes) * self.cfg["n_fast"]
        g = np.zeros(size) if grads else None
        loss = lib().orc_chunk_loss_grad(self.h, _ptr(x), len(x), _ptr(t) if len(t) else None, len(t),
                                         pos0, None if g is None else _ptr(g))
        if not grads:
            return loss, None
        out, o = [], 0
        for _ in range(self.cfg["n_fast"]):
            for shp in self.shapes:
                n = shp[0] * shp[1]
                out.append(g[o:o + n].reshape(shp))
                o += n
        return loss, out


def prefill(cfg, weights, tokens, chunk: int, lr: float, steps: int = 1, pos_offset: int = 0):
    """Whole-context inner loop; ``dict(losses, fast (canonical list), last_logits)``."""
    return CppOracle(cfg, weights).prefill(tokens, chunk, lr, steps, pos_offset)


def rope(x, pos, base: float = 10000.0, sign: int = 1):
    """RoPE of ``x [n, H, hd]`` at positions ``pos`` (sign -1: the transpose)."""
    a = np.ascontiguousarray(np.array(x, dtype=np.float64))
    p = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    n, H, hd = a.shape
    lib().orc_rope(_ptr(a), n, H, hd, _ptr(p), float(base), int(sign))
    return a


def layer_norm(x, eps: float):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    y = np.zeros_like(a)
    lib().orc_layer_norm(_ptr(a), a.shape[0], a.shape[1], float(eps), _ptr(y))
    return y


def attention(q, k, v, qpos, kpos, window: int):
    """Banded causal attention of ``q [nq,H,hd]`` over ``k, v [nk,H,hd]``."""
    q, k, v = (np.ascontiguousarray(np.asarray(a, dtype=np.float64)) for a in (q, k, v))
    qp = np.ascontiguousarray(np.asarray(qpos, dtype=np.int64))
    kp = np.ascontiguousarray(np.asarray(kpos, dtype=np.int64))
    o = np.zeros_like(q)
    lib().orc_attention(_ptr(q), _ptr(k), _ptr(v), q.shape[0], k.shape[0], q.shape[1], q.shape[2],
                        _ptr(qp), _ptr(kp), int(window), _ptr(o))
    return o
