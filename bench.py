"""Benchmark of the TTT-E2E inner loop on one MI355X.

One step = one whole prefill of the 3B-shape workload: 28 layers, d 3072,
24 heads of 128, SwiGLU 8192, vocab 32000, window 8192, T = 131072 tokens in
chunks of 1024, the MLPs of the last 7 blocks updated by SGD (lr 1e-4) after
every chunk.  Inputs are synthetic (Zipf(1.1) tokens with planted repeats
16K-64K apart, N(0, 0.02) weights rounded to bf16) and resident in HBM
before the timed region.

Prints one JSON line: prefill context tokens/s (value), decode ms/token
after the prefill (2048 greedy tokens, so two decode-time updates are
amortised in it), the MFMA utilisation of the whole prefill against the
bf16 dense peak, the roofline of the dominant kernel (HIP events around its
launches inside the timed region), the same context read without updates
(window 8192, and full attention with window = T: prefill and decode
latency against TTT-E2E's) and the float64 oracle's rate on the host cores
for a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch of the fused weight-gradient + SGD kernel from two
# rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) over the 3B-shape prefill,
# scaled by a plain 1 GiB elementwise copy measured in the same runs
# (FETCH_SIZE reads 0.5x the bytes read, WRITE_SIZE 1.0x the bytes written),
# averaged over the two launch shapes.  Valid only for the GEMM source it was
# measured on (sha256 of csrc/gemm.hip); otherwise reported as null.
SGD_TRAFFIC = {"gemm_src_sha256": "757c73ed1714f323c1667233b4ee441fba84acc2d61e9b30584ddb91be2b081c",
               "bytes_per_launch": 656.8e6,
               "profile": "profiles/sgd_gemm_3B_chunk1024_traffic.md"}


def _gemm_src_sha():
    import hashlib
    path = os.path.join(ROOT, "long_context_lm_chunk_amd", "csrc", "gemm.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def prefill_flops(cfg, T):
    """Algorithmic FLOPs of one prefill (forward of every layer, head,
    backward of the fast blocks; recomputation not counted)."""
    L, d, F, V, W, C, q = (cfg[k] for k in ("n_layers", "d_model", "d_ff", "vocab", "window",
                                            "chunk", "n_fast"))
    k = 3 if cfg["mlp"] == "swiglu" else 2
    sum_n = sum(min(t + 1, W) for t in range(T))
    sum_m = 0
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        sum_m += sum(min(u + 1, W) for u in range(n))
    fwd = 2 * (T * L * (4 * d * d + k * d * F) + L * d * 2 * sum_n + (T - 1) * d * V)
    bwd = 2 * ((T - 1) * d * V + T * (k + 1) * d * F + (q - 1) * T * (2 * k * d * F + 4 * d * d)
               + (q - 1) * d * (2 * sum_n + 2 * sum_m))
    if cfg.get("static_mlp"):
        # frozen second MLP of every fast block: its forward, and the two
        # input-gradient products of its backward (no weight gradient)
        fwd += 2 * T * q * k * d * F
        bwd += 2 * T * q * k * d * F
    return float(fwd + bwd)


def forward_flops(cfg, T):
    """Algorithmic FLOPs of one read of the context without updates (every
    layer's forward and the head)."""
    L, d, F, V, W = (cfg[k] for k in ("n_layers", "d_model", "d_ff", "vocab", "window"))
    k = 3 if cfg["mlp"] == "swiglu" else 2
    sum_n = sum(min(t + 1, W) for t in range(T))
    extra = 2 * T * cfg["n_fast"] * k * d * F if cfg.get("static_mlp") else 0
    return float(2 * (T * L * (4 * d * d + k * d * F) + L * d * 2 * sum_n + (T - 1) * d * V) + extra)


def sgd_bytes_per_launch(cfg, T, per_weight=10.0):
    """Algorithmic HBM bytes of one fused weight-gradient + SGD launch,
    averaged over the launches of a prefill: per fast weight the SGD step's
    own traffic, an fp32 master read and written and a bf16 copy written for
    the next forward (10 B), plus both bf16 operands ([out][tokens] and
    [in][tokens], tokens padded to 8).  per_weight=14 gives the design's
    bytes: it also reads W0 (2 B) and writes the transposed current weight
    round(W0 + delta) (2 B) for the input-gradient products."""
    d, F, C = cfg["d_model"], cfg["d_ff"], cfg["chunk"]
    F2 = 2 * F if cfg["mlp"] == "swiglu" else F
    tot, launches = 0.0, 0
    for c0 in range(0, T - 1, C):
        n = min(C, T - c0)
        np_ = (n + 7) // 8 * 8
        for (M, N) in ((d, F), (F2, d)):
            tot += per_weight * M * N + 2.0 * (M + N) * np_
            launches += 1
    return tot / max(launches, 1)


def sgd_flops_per_launch(cfg, T):
    d, F, C = cfg["d_model"], cfg["d_ff"], cfg["chunk"]
    F2 = 2 * F if cfg["mlp"] == "swiglu" else F
    tot, launches = 0.0, 0
    for c0 in range(0, T - 1, C):
        n = min(C, T - c0)
        tot += 2.0 * (d * F + F2 * d) * n
        launches += 2
    return tot / max(launches, 1)


def cpu_baseline(cfg, weights_gpu, tokens_np, sample_tokens=256):
    """The float64 oracle on the host cores: the first `sample_tokens` tokens
    of the workload read as one chunk (forward through every layer, CE,
    backward through the fast blocks, SGD)."""
    import numpy as np
    import torch
    from oracle import ttt_oracle as O
    w = [t.cpu() for t in weights_gpu]
    model = O.OracleModel(cfg, w)
    del w
    threads = torch.get_num_threads()
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 0) for i in info] + [1])
    except Exception:
        pass
    x = tokens_np[:sample_tokens + 1]
    t0 = time.perf_counter()
    O.prefill(cfg, None, x[:sample_tokens], sample_tokens, cfg["lr"], model=model)
    dt = time.perf_counter() - t0
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of the workload as one chunk "
                      f"({dt:.1f} s; attention windows <= {sample_tokens} keys, so this overstates "
                      f"the oracle's steady-state rate)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c4")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--decode-tokens", type=int, default=2048,
                    help="greedy decode tokens timed after the prefill (2048 reach two "
                         "decode-time updates at chunk 1024)")
    ap.add_argument("--decode-sweep", default="8192,32768,131072,524288",
                    help="comma-separated prefill lengths after each of which 256 decode tokens are "
                         "timed (decode cost against context length); empty to skip")
    ap.add_argument("--contexts", type=int, default=1,
                    help="also time this many independent contexts prefilled at once "
                         "(one model each, chains interleaved on their own streams)")
    ap.add_argument("--static-mlp", action="store_true",
                    help="the variant whose fast blocks also carry a frozen second MLP")
    ap.add_argument("--no-static", action="store_true",
                    help="skip the reads without updates (window 8192, and full attention)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=1024)
    ap.add_argument("--prefill-block", type=int, default=0,
                    help="tokens per batched pass over the frozen blocks (0: the library default)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="MiB of a plain device copy run first, as the reference for "
                         "FETCH_SIZE/WRITE_SIZE counter scaling")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the inner loop of one "
              "context is sequential over chunks and this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    if args.contexts > 1:
        # every context brings its own four streams: enough hardware queues
        # for them not to share one (set before the runtime starts)
        os.environ.setdefault("GPU_MAX_HW_QUEUES", str(min(32, 4 * args.contexts + 2)))
    import numpy as np
    import torch
    import synth
    import long_context_lm_chunk_amd as T_

    cfg = synth.config(args.config)
    if args.static_mlp:
        cfg = synth.config(cfg, static_mlp=1, name=cfg["name"] + "+static-second-MLP")
    T = args.T or cfg["T"]
    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()
    weights = synth.gen_weights(cfg, device=dev)
    tokens_np = synth.gen_tokens(cfg, T=T)
    tokens = torch.from_numpy(tokens_np).to(dev)
    model = T_.Model(cfg, weights, max_chunk=cfg["chunk"], prefill_block=args.prefill_block)
    torch.cuda.synchronize()
    print(f"# setup {time.perf_counter() - t_setup:.1f}s, workspace "
          f"{model.workspace.numel() / 1e9:.2f} GB", file=sys.stderr, flush=True)

    if args.copy_probe:
        src = torch.ones(args.copy_probe * (1 << 18), dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)   # one elementwise kernel: N*4 bytes read, N*4 written
        torch.cuda.synchronize()
        print(f"# copy probe: {args.copy_probe} MiB read + {args.copy_probe} MiB written",
              file=sys.stderr, flush=True)
        del src, dst

    losses = None
    for i in range(args.warmup):
        losses = model.prefill(tokens, cfg["chunk"], cfg["lr"])
        torch.cuda.synchronize()
        print(f"# warmup {i} done", file=sys.stderr, flush=True)

    # kernel classes timed with HIP events on the streams they run on; the
    # dominant kernel (the fused weight-gradient + SGD products) is class 4
    classes = {0: "gemm_all", 1: "attn_fwd", 2: "attn_bwd", 3: "head_ce", 4: "dw_sgd", 5: "mlp_up"}
    for c in classes:
        model.timing_enable(c, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        losses = model.prefill(tokens, cfg["chunk"], cfg["lr"])
        print(f"# step {i} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ktime = {}
    for c, name in classes.items():
        ms, n, fl = model.timing_read(c)
        ktime[name] = dict(ms=ms / args.steps, launches=n // args.steps, flops=fl / args.steps)
        model.timing_enable(c, False)
    ms_per_step = dt * 1000.0 / args.steps
    tok_s = T / (dt / args.steps)
    fl = prefill_flops(dict(cfg, T=T), T)
    mfma_pct = 100.0 * fl / (dt / args.steps) / (PEAK_BF16_TFLOPS * 1e12)
    print("# kernel classes per step: " + ", ".join(
        f"{k} {v['ms']:.1f} ms/{v['launches']} launches/"
        f"{(v['flops'] / max(v['ms'], 1e-9) / 1e9) if v['flops'] else 0:.0f} TF/s"
        for k, v in ktime.items()), file=sys.stderr, flush=True)
    lh = losses.cpu().numpy()
    assert np.all(np.isfinite(lh)), "non-finite chunk loss"

    # decode after the prefill (constant per-token cost once T >= window); the
    # decode-time updates fire when 1024 decode positions are complete, each
    # token is bracketed by events so update tokens are seen separately
    def timed_decode(mdl, n, ctx=None):
        for _ in range(4):
            mdl.decode_step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        uls = []
        ev[0].record()
        for i in range(n):
            uls.append(mdl.decode_step()[2])
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
        upd = np.array([not bool(torch.isnan(u).item()) for u in uls])
        res = {"tokens": n, "ms_per_token": round(float(per.sum() / n), 4),
               "ms_per_token_p50": round(float(np.percentile(per, 50)), 4),
               "ms_per_token_p99": round(float(np.percentile(per, 99)), 4),
               "updates": int(upd.sum()),
               "update_token_ms": round(float(per[upd].mean()), 3) if upd.any() else None,
               "ms_per_token_without_updates": round(float(per[~upd].mean()), 4) if (~upd).any() else None,
               "first_position": int((T if ctx is None else ctx) + 4)}
        return res

    dec = None
    if args.decode_tokens > 0:
        dec = timed_decode(model, args.decode_tokens)
        print(f"# decode: {dec}", file=sys.stderr, flush=True)

    # The matrix cores' own peak on this GPU (bf16 products from registers)
    # and the shader clock they ran at, beside the specified peak.
    mpeak = None
    try:
        tf, mhz = T_.diag_mfma_peak()
        mpeak = {"tflops": round(tf, 1), "clock_mhz": round(mhz, 0),
                 "mfma_util_pct_of_measured_peak": round(100.0 * fl / (dt / args.steps) / (tf * 1e12), 2)}
        print(f"# measured bf16 matrix-core peak: {mpeak}", file=sys.stderr, flush=True)
    except Exception as e:   # noqa: BLE001
        mpeak = {"error": f"{type(e).__name__}: {e}"}
    # and the HBM rate of a plain 2 GiB device copy (read + write), beside
    # the specified 8 TB/s
    try:
        src = torch.ones(1 << 29, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ce0.record()
        for _ in range(10):
            dst.copy_(src)
        ce1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * src.numel() * 4 * 10 / (ce0.elapsed_time(ce1) / 1e3) / 1e9
        mpeak = dict(mpeak or {}, hbm_copy_gbs=round(copy_gbs, 1))
        del src, dst
        torch.cuda.empty_cache()
    except Exception as e:   # noqa: BLE001
        mpeak = dict(mpeak or {}, hbm_copy_error=f"{type(e).__name__}: {e}")

    # Decode cost against the context length read before it.
    sweep = None
    if args.decode_sweep:
        try:
            sweep = []
            for Ts in [int(v) for v in args.decode_sweep.split(",")]:
                tk = torch.from_numpy(synth.gen_tokens(cfg, T=Ts)).to(dev)
                model.prefill(tk, cfg["chunk"], cfg["lr"])
                r = timed_decode(model, 256, Ts)
                sweep.append({"T": Ts, "ms_per_token": r["ms_per_token"], "p50": r["ms_per_token_p50"],
                              "p99": r["ms_per_token_p99"]})
                print(f"# decode after T={Ts}: {sweep[-1]}", file=sys.stderr, flush=True)
                del tk
        except Exception as e:   # noqa: BLE001
            sweep = {"error": f"{type(e).__name__}: {e}"}

    # Several independent contexts prefilled at once (one model each: own
    # fast weights and rings; the same weights, other token seeds).
    multi = None
    if args.contexts > 1:
        # an optional leg: a failure is reported in the line, the headline
        # figures above stand
        try:
            extra = [T_.Model(cfg, weights, max_chunk=cfg["chunk"], prefill_block=args.prefill_block)
                     for _ in range(args.contexts - 1)]
            mods = [model] + extra
            toks = [tokens] + [torch.from_numpy(synth.gen_tokens(cfg, T=T, seed=cfg["token_seed"] + 1000 + i))
                               .to(dev) for i in range(args.contexts - 1)]
            T_.prefill_many(mods, toks, cfg["chunk"], cfg["lr"])
            torch.cuda.synchronize()
            reps = 2
            t0 = time.perf_counter()
            for _ in range(reps):
                outs = T_.prefill_many(mods, toks, cfg["chunk"], cfg["lr"])
            torch.cuda.synchronize()
            t_m = (time.perf_counter() - t0) / reps
            assert all(bool(torch.isfinite(o).all().item()) for o in outs), "non-finite loss (contexts)"
            multi = {"contexts": args.contexts, "ms": round(t_m * 1e3, 1),
                     "tokens_per_s": round(args.contexts * T / t_m, 1),
                     "speedup_over_one_context": round(args.contexts * (dt / args.steps) / t_m, 3)}
            print(f"# {args.contexts} contexts at once: {multi}", file=sys.stderr, flush=True)
            for e in extra:
                e.close()
            del extra, mods, toks
            torch.cuda.empty_cache()
        except Exception as e:   # noqa: BLE001
            multi = {"error": f"{type(e).__name__}: {e}"}
            print(f"# contexts leg failed: {multi['error']}", file=sys.stderr, flush=True)

    # The same context read without updates (the static-weight models the
    # pages compare TTT-E2E with): window 8192, then full attention (window
    # = T), prefill and decode latency.
    static = None
    if not args.no_static:
        try:
            def timed_forward(mdl, reps):
                mdl.forward(tokens, cfg["chunk"])
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(reps):
                    out = mdl.forward(tokens, cfg["chunk"])
                torch.cuda.synchronize()
                assert bool(torch.isfinite(out).all().item()), "non-finite loss in the static read"
                return (time.perf_counter() - t0) / reps
            t_sw = timed_forward(model, 2)
            print(f"# static read, window {cfg['window']}: {t_sw * 1e3:.1f} ms", file=sys.stderr, flush=True)
            model.close()
            del model
            torch.cuda.empty_cache()
            fcfg = synth.config(cfg, window=T)
            fa = T_.Model(fcfg, weights, max_chunk=cfg["chunk"], prefill_block=args.prefill_block)
            print(f"# full-attention model: workspace {fa.workspace.numel() / 1e9:.1f} GB", file=sys.stderr,
                  flush=True)
            t_fa = timed_forward(fa, 2)
            print(f"# full-attention read: {t_fa * 1e3:.1f} ms", file=sys.stderr, flush=True)
            fdec = timed_decode(fa, 64) if args.decode_tokens > 0 else None
            fa.close()
            del fa
            torch.cuda.empty_cache()
            ttt_s = dt / args.steps
            static = {
                "T": T,
                "window_static": {"window": cfg["window"], "ms": round(t_sw * 1e3, 1),
                                  "tokens_per_s": round(T / t_sw, 1),
                                  "mfma_util_pct": round(100.0 * forward_flops(cfg, T) / t_sw /
                                                         (PEAK_BF16_TFLOPS * 1e12), 2)},
                "full_attention": {"window": T, "ms": round(t_fa * 1e3, 1), "tokens_per_s": round(T / t_fa, 1),
                                   "mfma_util_pct": round(100.0 * forward_flops(fcfg, T) / t_fa /
                                                          (PEAK_BF16_TFLOPS * 1e12), 2),
                                   "decode_ms_per_token": fdec["ms_per_token"] if fdec else None},
                "prefill_latency_ratio_full_attention_over_ttt": round(t_fa / ttt_s, 3),
                "decode_latency_ratio_full_attention_over_ttt": (round(fdec["ms_per_token_without_updates"] /
                                                                       dec["ms_per_token_without_updates"], 3)
                                                                 if fdec and dec else None),
            }
        except Exception as e:   # noqa: BLE001
            static = {"error": f"{type(e).__name__}: {e}"}
            print(f"# static-read leg failed: {static['error']}", file=sys.stderr, flush=True)

    # Roofline of the dominant kernel (largest measured time of the classes
    # that are one kernel symbol each): the fused weight-gradient + SGD
    # products (bound by HBM: ~140 FLOP per byte, below the ridge point of
    # 2.5 PFLOP/s / 8 TB/s) or the frozen-block MLP up-projection (MFMA).
    roof = None
    sg, up = ktime["dw_sgd"], ktime["mlp_up"]
    if sg["launches"] and (sg["ms"] >= up["ms"] or not up["launches"]):
        avg_ms = sg["ms"] / sg["launches"]
        by = sgd_bytes_per_launch(dict(cfg, T=T), T)
        by_design = sgd_bytes_per_launch(dict(cfg, T=T), T, per_weight=14.0)
        ach = by / (avg_ms / 1e3) / 1e9
        traffic = (SGD_TRAFFIC["bytes_per_launch"] if _gemm_src_sha() == SGD_TRAFFIC["gemm_src_sha256"]
                   else None)
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": "gemm256_kernel<SGD epilogue, bf16> (fused weight gradient + SGD of the "
                          "fast MLPs: [d][F] and [2F][d] over the chunk's tokens, 256x256 tiles)",
                "algorithmic_bytes_per_launch": round(by),
                "algorithmic_bytes_rule": "10 B per fast weight (fp32 master read + write, bf16 copy write) "
                                          "+ both bf16 operands",
                "design_bytes_per_launch": round(by_design),
                "design_gbs": round(by_design / (avg_ms / 1e3) / 1e9, 1),
                "flops_per_launch": round(sgd_flops_per_launch(dict(cfg, T=T), T)),
                "avg_launch_ms": round(avg_ms, 4), "launches_per_step": sg["launches"],
                "stream": "fast-weight update stream (concurrent with the backward chain)"}
    elif up["launches"]:
        avg_ms = up["ms"] / up["launches"]
        ach = up["flops"] / up["launches"] / (avg_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "kernel": "gemm256_kernel<SWIGLU, bf16, single B> (frozen-block MLP up-projection, "
                          "M=8192 N=16384 K=3072)",
                "avg_launch_ms": round(avg_ms, 4), "launches_per_step": up["launches"]}

    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, weights, tokens_np, args.cpu_sample)

    out = {
        "metric": ("TTT-E2E prefill context tokens/s at 3B/128K; decode ms/token; MFMA util %"
                   if args.config == "c4" and T == 131072 and not args.static_mlp else
                   f"TTT-E2E prefill context tokens/s ({cfg['name']}, T={T}); decode ms/token; MFMA util %"),
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (Zipf(1.1) tokens with planted repeats; N(0,0.02) weights, bf16)",
        "config": {"workload": f"ttt-e2e prefill, {cfg['name']}", "T": T, "chunk": cfg["chunk"],
                   "window": cfg["window"], "layers": cfg["n_layers"], "d_model": cfg["d_model"],
                   "heads": cfg["n_heads"], "d_ff": cfg["d_ff"], "vocab": cfg["vocab"],
                   "fast_layers": cfg["n_fast"], "lr": cfg["lr"], "steps_per_chunk": 1,
                   "static_second_mlp": bool(cfg.get("static_mlp", 0)),
                   "parallelism": "single GPU"},
        "decode_ms_per_token": None if dec is None else dec["ms_per_token"],
        "decode": dec,
        "static_reads": static,
        "contexts_at_once": multi,
        "decode_by_context_length": sweep,
        "mfma_util_pct": round(mfma_pct, 2),
        "mfma_peak_measured": mpeak,
        "algorithmic_tflop_per_step": round(fl / 1e12, 1),
        "kernel_classes_ms_per_step": {k: round(v["ms"], 2) for k, v in ktime.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "mean_chunk_loss": float(lh.mean()),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
