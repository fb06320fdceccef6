"""MI355X-native TTT-E2E test-time inner loop (End-to-End Test-Time Training
for Long Context).

Python binding of ``libttt.so`` (C ABI in ``include/ttt.h``).  This module
only marshals arguments: torch provides device memory and the stream, every
step of the inner loop runs in the library's HIP kernels.  There is no CPU
fallback: if the library is missing, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["lib", "TTTConfig", "Model", "TTTError", "config_from_dict", "LIB_PATH", "prefill_many"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttt.so")

TTT_MLP_GELU, TTT_MLP_SWIGLU = 0, 1
TTT_FP32, TTT_BF16 = 0, 1


class TTTError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"ttt status {status}: {msg}")
        self.status = status


class TTTConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("window", ctypes.c_int32), ("n_fast", ctypes.c_int32), ("mlp", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_float), ("ln_eps", ctypes.c_float),
        ("max_chunk", ctypes.c_int32), ("prefill_block", ctypes.c_int32),
        ("static_mlp", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python long_context_lm_chunk_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sig = {
        "ttt_workspace_bytes": ([ctypes.POINTER(TTTConfig), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
        "ttt_model_load": ([ctypes.POINTER(TTTConfig), ctypes.POINTER(vp), i32, vp, ctypes.c_size_t, vp,
                            ctypes.POINTER(vp)], ctypes.c_int),
        "ttt_model_load_static": ([ctypes.POINTER(TTTConfig), ctypes.POINTER(vp), i32, vp, ctypes.POINTER(vp)],
                                  ctypes.c_int),
        "ttt_prefill": ([vp, vp, i64, i32, f32, i32, vp, vp], ctypes.c_int),
        "ttt_forward": ([vp, vp, i64, i32, vp, vp], ctypes.c_int),
        "ttt_prefill_many": ([ctypes.POINTER(vp), i32, ctypes.POINTER(vp), i64, i32, f32, i32,
                              ctypes.POINTER(vp), vp], ctypes.c_int),
        "ttt_fast_weight": ([vp, i32, i32, vp, i64, vp], ctypes.c_int),
        "ttt_fast_weight_delta": ([vp, i32, i32, vp, i64, vp], ctypes.c_int),
        "ttt_decode_step": ([vp, vp, vp, vp, vp], ctypes.c_int),
        "ttt_reset": ([vp, vp], ctypes.c_int),
        "ttt_model_free": ([vp], None),
        "ttt_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "ttt_last_error": ([], ctypes.c_char_p),
        "ttt_timing_enable": ([vp, i32, i32], ctypes.c_int),
        "ttt_timing_read": ([vp, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64),
                             ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "ttt_diag_gemm": ([i32, i32, i32, i32, i32, i32, vp, i64, vp, i64, vp, i64, vp], ctypes.c_int),
        "ttt_diag_gemm_core": ([i32], ctypes.c_int),
        "ttt_diag_chunk_logits": ([vp, vp, i64, vp], ctypes.c_int),
        "ttt_diag_chunk_logit_rows": ([vp], i64),
        "ttt_diag_sgd": ([i32, i32, i32, i32, vp, i64, vp, i64, f32, vp, vp, vp, vp, vp], ctypes.c_int),
        "ttt_diag_mfma_peak": ([vp, vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), vp],
                               ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


lib = _load()

EXPORTED = ["ttt_workspace_bytes", "ttt_model_load", "ttt_model_load_static", "ttt_prefill", "ttt_forward", "ttt_prefill_many", "ttt_fast_weight",
            "ttt_fast_weight_delta",
            "ttt_decode_step", "ttt_reset", "ttt_model_free", "ttt_status_str", "ttt_last_error",
            "ttt_timing_enable", "ttt_timing_read", "ttt_diag_gemm", "ttt_diag_gemm_core",
            "ttt_diag_sgd", "ttt_diag_chunk_logits", "ttt_diag_chunk_logit_rows", "ttt_diag_mfma_peak"]


GEMM_CORE_AUTO, GEMM_CORE_BIG, GEMM_CORE_SMALL = 0, 1, 2


def diag_gemm_core(mode: int) -> int:
    """Select the GEMM core for bf16 k-contiguous products (see
    ttt_diag_gemm_core); returns the previous mode."""
    return int(lib.ttt_diag_gemm_core(int(mode)))


def diag_mfma_peak():
    """(TFLOP/s, MHz): bf16 matrix-core throughput from registers and the
    shader clock it ran at, measured on the current device."""
    import torch
    scratch = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    tf, mhz = ctypes.c_double(0), ctypes.c_double(0)
    s = torch.cuda.current_stream()
    _check(lib.ttt_diag_mfma_peak(ctypes.c_void_p(scratch.data_ptr()), ctypes.c_void_p(clk.data_ptr()),
                                  ctypes.byref(tf), ctypes.byref(mhz), ctypes.c_void_p(s.cuda_stream)))
    return tf.value, mhz.value


def diag_gemm(A, B, M, N, K, a_kc: bool, b_kc: bool, C=None):
    """C = A.B through the library's GEMM kernel (see ttt_diag_gemm)."""
    import torch
    dt = TTT_BF16 if A.dtype == torch.bfloat16 else TTT_FP32
    if C is None:
        C = torch.zeros(M, N, dtype=torch.float32, device=A.device)
    lda = A.shape[1]
    ldb = B.shape[1]
    s = torch.cuda.current_stream(A.device).cuda_stream
    _check(lib.ttt_diag_gemm(dt, int(a_kc), int(b_kc), M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                             C.data_ptr(), C.shape[1], s))
    return C


def diag_sgd(A, B, lr: float, master, w0):
    """The fused weight-gradient + SGD product on A [M][K], B [N][K] (see
    ttt_diag_sgd): updates ``master`` [M][N] (float32) in place and returns
    (copy [M][N] or None, cur_t [N][M]) in the element type of A."""
    import torch
    M, K = A.shape
    N = B.shape[0]
    bf = A.dtype == torch.bfloat16
    copy = torch.empty(M, N, dtype=A.dtype, device=A.device) if bf else None
    cur_t = torch.empty(N, M, dtype=A.dtype, device=A.device)
    s = torch.cuda.current_stream(A.device).cuda_stream
    _check(lib.ttt_diag_sgd(TTT_BF16 if bf else TTT_FP32, M, N, K, A.data_ptr(), A.stride(0), B.data_ptr(),
                            B.stride(0), float(lr), master.data_ptr(), copy.data_ptr() if bf else None,
                            w0.data_ptr(), cur_t.data_ptr(), s))
    return copy, cur_t


def _check(rc: int):
    if rc != 0:
        raise TTTError(rc, lib.ttt_last_error().decode())


def config_from_dict(cfg: dict, max_chunk: int | None = None, prefill_block: int = 0,
                     dtype: str | None = None) -> TTTConfig:
    """Map a workload dict (``synth.config``) onto the C struct."""
    dt = cfg["dtype"] if dtype is None else dtype
    return TTTConfig(
        n_layers=cfg["n_layers"], d_model=cfg["d_model"], n_heads=cfg["n_heads"],
        head_dim=cfg["head_dim"], d_ff=cfg["d_ff"], vocab=cfg["vocab"], window=cfg["window"],
        n_fast=cfg["n_fast"], mlp=TTT_MLP_SWIGLU if cfg["mlp"] == "swiglu" else TTT_MLP_GELU,
        dtype=TTT_BF16 if dt == "bf16" else TTT_FP32, rope_base=cfg.get("rope_base", 10000.0),
        ln_eps=cfg.get("ln_eps", 1e-5), max_chunk=max_chunk or cfg["chunk"],
        prefill_block=prefill_block, static_mlp=int(bool(cfg.get("static_mlp", 0))))


def workspace_bytes(c: TTTConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.ttt_workspace_bytes(ctypes.byref(c), ctypes.byref(n)))
    return n.value


def prefill_many(models, tokens_list, chunk: int, lr: float, steps: int = 1, stream=None):
    """The inner loop over several independent contexts at once, one model
    per context (see ttt_prefill_many); returns each context's losses."""
    import torch
    if len(models) != len(tokens_list) or not models:
        raise ValueError("one token tensor per model")
    dev = models[0].device
    toks = [t.to(dev, torch.int32).contiguous() for t in tokens_list]
    T = toks[0].numel()
    if any(t.numel() != T for t in toks):
        raise ValueError("every context must have the same length")
    outs = [torch.empty(math.ceil(T / chunk) * steps, dtype=torch.float32, device=dev) for _ in models]
    n = len(models)
    hs = (ctypes.c_void_p * n)(*[m.h.value for m in models])
    tp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in toks])
    lp = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _check(lib.ttt_prefill_many(hs, n, tp, T, chunk, float(lr), steps, lp, ctypes.c_void_p(s.cuda_stream)))
    return outs


class Model:
    """A loaded model: torch owns the workspace; the library owns nothing on
    the device."""

    def __init__(self, cfg: dict, weights, dtype: str | None = None, max_chunk: int | None = None,
                 prefill_block: int = 0, stream=None, static_workspace: bool = False):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.c = config_from_dict(cfg, max_chunk=max_chunk, prefill_block=prefill_block, dtype=dtype)
        self.dtype = torch.bfloat16 if self.c.dtype == TTT_BF16 else torch.float32
        self.device = weights[0].device
        if self.device.type != "cuda":
            raise ValueError("weights must be device (cuda/HIP) tensors")
        ws_weights = [w.to(self.dtype).contiguous() for w in weights]
        ptrs = (ctypes.c_void_p * len(ws_weights))(*[w.data_ptr() for w in ws_weights])
        h = ctypes.c_void_p(0)
        self._stream = stream
        if static_workspace:
            # device state in the library's static array (ttt_model_load_static)
            self.workspace = None
            with torch.cuda.device(self.device):
                _check(lib.ttt_model_load_static(ctypes.byref(self.c), ptrs, len(ws_weights), self._s(),
                                                 ctypes.byref(h)))
        else:
            ws = workspace_bytes(self.c)
            self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
            _check(lib.ttt_model_load(ctypes.byref(self.c), ptrs, len(ws_weights),
                                      self.workspace.data_ptr(), ws, self._s(), ctypes.byref(h)))
        self.h = h
        del ws_weights

    def _s(self):
        s = self._stream if self._stream is not None else self.torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(s.cuda_stream)

    def prefill(self, tokens, chunk: int, lr: float, steps: int = 1, out=None):
        torch = self.torch
        tokens = tokens.to(self.device, torch.int32).contiguous()
        T = tokens.numel()
        n = math.ceil(T / chunk) * steps
        if out is None:
            out = torch.empty(n, dtype=torch.float32, device=self.device)
        _check(lib.ttt_prefill(self.h, tokens.data_ptr(), T, chunk, float(lr), steps,
                               out.data_ptr(), self._s()))
        return out

    def forward(self, tokens, chunk: int, out=None):
        """The context read with the loaded weights and no update (per-chunk
        losses as a prefill at lr = 0); with window >= T, full attention."""
        torch = self.torch
        tokens = tokens.to(self.device, torch.int32).contiguous()
        T = tokens.numel()
        if out is None:
            out = torch.empty(math.ceil(T / chunk), dtype=torch.float32, device=self.device)
        _check(lib.ttt_forward(self.h, tokens.data_ptr(), T, chunk, out.data_ptr(), self._s()))
        return out

    def fast_weight(self, fast_idx: int, mat: int, delta: bool = False):
        """Fast matrix `mat` of fast layer `fast_idx`, float32 [in][out];
        with delta, its change since loading (exact float32 master)."""
        torch = self.torch
        d, F = self.cfg["d_model"], self.cfg["d_ff"]
        nmat = 3 if self.cfg["mlp"] == "swiglu" else 2
        shape = (F, d) if mat == nmat - 1 else (d, F)
        out = torch.empty(shape, dtype=torch.float32, device=self.device)
        fn = lib.ttt_fast_weight_delta if delta else lib.ttt_fast_weight
        _check(fn(self.h, fast_idx, mat, out.data_ptr(), out.numel(), self._s()))
        return out

    def fast_weights(self, delta: bool = False):
        nmat = 3 if self.cfg["mlp"] == "swiglu" else 2
        return [self.fast_weight(j, m, delta) for j in range(self.cfg["n_fast"]) for m in range(nmat)]

    def decode_step(self, want_logits: bool = False):
        torch = self.torch
        tok = torch.empty(1, dtype=torch.int32, device=self.device)
        lg = torch.empty(self.cfg["vocab"], dtype=torch.float32, device=self.device) if want_logits else None
        ul = torch.empty(1, dtype=torch.float32, device=self.device)
        _check(lib.ttt_decode_step(self.h, tok.data_ptr(), lg.data_ptr() if lg is not None else None,
                                   ul.data_ptr(), self._s()))
        return tok, lg, ul

    def chunk_logits(self):
        """Logits [rows][vocab] of the last chunk read with updates (see
        ttt_diag_chunk_logits)."""
        torch = self.torch
        rows = int(lib.ttt_diag_chunk_logit_rows(self.h))
        out = torch.empty(rows, self.cfg["vocab"], dtype=torch.float32, device=self.device)
        _check(lib.ttt_diag_chunk_logits(self.h, out.data_ptr(), out.numel(), self._s()))
        return out

    def reset(self):
        _check(lib.ttt_reset(self.h, self._s()))

    def timing_enable(self, cls: int, on: bool = True):
        _check(lib.ttt_timing_enable(self.h, cls, int(on)))

    def timing_read(self, cls: int):
        ms = ctypes.c_double(0)
        n = ctypes.c_int64(0)
        fl = ctypes.c_double(0)
        _check(lib.ttt_timing_read(self.h, cls, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl)))
        return ms.value, n.value, fl.value

    def close(self):
        if getattr(self, "h", None) is not None and self.h.value:
            lib.ttt_model_free(self.h)
            self.h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
