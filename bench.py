#!/usr/bin/env python3
"""Training-step throughput of the depth-parameterised GPT on one MI355X.

One step = gpt_fwd_bwd (embedding, blocks, head + cross-entropy, full
backward) + muon_step (momentum, Newton-Schulz, update of every block matrix)
+ adamw_step (wte and lm_head) on one microbatch of seeded synthetic tokens,
with inputs and weights resident in HBM before the timed region. With
--accum K a step runs K microbatches (gradient accumulation) before the two
optimizer calls; with --normuon the block matrices take normuon_step (Muon
with NorMuon variance reduction, beta2 0.95) in place of muon_step. Prints one
JSON line:

  value        training tokens/s (B*T*steps / wall time of the timed steps)
  mfu          value * F_tok / MI355X dense-bf16 peak, with
               F_tok = 6 (12 L d^2 + V d) + 6 L d T (causal attention once)
  roofline     the GEMM kernel family (the dominant kernel): algorithmic FLOPs
               of its launches / their summed durations, from HIP events
               recorded around each launch on its stream during a second timed
               pass of the same steps (the headline pass runs without them)
  measured_peaks  the MFMA rate and copy bandwidth measured on this GPU
  cpu_baseline the CPU oracle on a bounded sample of the same workload

Metric definitions follow the page's train/mfu and train/tok_per_sec
("Como treinar seu próprio ChatGPT por 50 dólares", section "Métricas para
Monitorar"); the page prints no value for them.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

from gpt_pretraining_step_bf16_amd import synthetic as syn

PEAK_BF16_FLOPS = 2.5166e15  # MI355X dense bf16 MFMA
METRIC = "training tokens/sec + MFU, d20 GPT fwd+bwd+Muon step on 1 MI355X"
# AdamW hyperparameters for wte / lm_head: the page names the optimizer only.
# PyTorch's default betas and eps, no decay, and a rate well below the 0.02
# init scale (early Adam steps move every element by about lr).
ADAMW = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
# NorMuon second-moment decay (the pages give none; the NorMuon method's usual value).
NORMUON_BETA2 = 0.95


def flops_per_token(L, d, V, T, windows=None, dkv=None):
    """Model FLOPs per token; causal attention counts T per layer (half of the
    T^2 score matrix, fwd+bwd). A windowed layer counts 2 * (visible pairs) / T.
    dkv: width of the key/value projections (d unless grouped-query)."""
    dkv = d if dkv is None else dkv
    att = 0.0
    for l in range(L):
        w = -1 if windows is None else windows[l]
        if w < 0 or w >= T - 1:
            att += T
        else:
            pairs = 0.5 * (w + 1) * (w + 2) + (T - 1 - w) * (w + 1)
            att += 2.0 * pairs / T
    return 6.0 * (L * (10.0 * d * d + 2.0 * dkv * d) + V * d) + 6.0 * d * att


def gemm_bytes_per_step(L, d, V, N, chunk, dkv=None):
    """Algorithmic HBM bytes of the fwd/bwd GEMM launches of one step: bf16 operands
    read once, outputs written once (fp32 for dX feeding a norm, for weight
    gradients and for the residual stream), epilogue operands (the fp32 residual,
    relu^2 activations) read once. The qkv width is d + 2 dkv."""
    F = 4 * d
    Q = d + 2 * (d if dkv is None else dkv)
    layer = (N * d * 2 + Q * d * 2 + N * Q * 2                    # QKV
             + N * d * 2 + d * d * 2 + 2 * N * d * 4              # O + fp32 residual
             + N * d * 2 + F * d * 2 + N * F * 2                  # FC, relu^2
             + N * F * 2 + F * d * 2 + 2 * N * d * 4              # proj + fp32 residual
             + N * d * 2 + d * F * 2 + 2 * N * F * 2              # dH, relu^2' epilogue
             + N * d * 2 + N * F * 2 + F * d * 4                  # dW_proj
             + N * F * 2 + F * d * 2 + N * d * 4                  # dXn2
             + N * F * 2 + N * d * 2 + F * d * 4                  # dW_fc
             + N * d * 2 + d * d * 2 + N * d * 2                  # dO
             + 2 * N * d * 2 + d * d * 4                          # dWo
             + N * Q * 2 + Q * d * 2 + N * d * 4                  # dXn
             + N * Q * 2 + N * d * 2 + Q * d * 4)                 # dW_qkv
    nchunks = -(-N // chunk)
    head = nchunks * ((chunk * d * 2 + V * d * 2 + chunk * V * 2)
                      + (chunk * V * 2 + V * d * 2 + chunk * d * 4)
                      + (chunk * V * 2 + chunk * d * 2 + 2 * V * d * 4))
    return L * layer + head, 12 * L + 3 * nchunks


def ns_flops(L, d, steps=5, dkv=None):
    # Per iteration, an r x c matrix (r >= c) costs 4 r c^2 + 2 c^3: the Gram
    # matrix, its square and the update. Per layer: wq, wo (d x d, 6 d^3 each),
    # wk, wv (d x dkv once oriented tall), wfc and wproj (4d x d, 18 d^3 each).
    dkv = d if dkv is None else dkv
    kv = 4.0 * d * dkv ** 2 + 2.0 * dkv ** 3
    return steps * L * (2 * 6.0 * d ** 3 + 2 * kv + 2 * 18.0 * d ** 3)


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "gemm_fwd_bwd_d20_hbm_traffic.txt")


def gemm_traffic():
    """HBM bytes per launch of the fwd/bwd GEMM family from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None when the GEMM sources changed since."""
    from gpt_pretraining_step_bf16_amd.profile_summary import gemm_source_hash

    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith("#"))
    if vals.get("source_sha256", "").strip() != gemm_source_hash():
        return None
    return float(vals["traffic_bytes_per_launch"])


def measured_peaks(torch):
    """Second denominators measured on this GPU: the dense-bf16 MFMA rate the
    chip sustains (the library's register-only MFMA probe, best of 3) and the
    bandwidth of a plain 1 GiB device copy (best of 5)."""
    from gpt_pretraining_step_bf16_amd import binding

    blocks, iters = 2048, 20000
    sink = torch.empty(blocks, dtype=torch.float32, device="cuda")
    best = 0.0
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fl = binding.probe_mfma_bf16(blocks, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, fl / (e0.elapsed_time(e1) / 1e3) / 1e12)
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    bw = 0.0
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        bw = max(bw, 2.0 * n * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del src, dst
    return {"mfma_bf16_tflops": round(best, 1), "copy_gbs": round(bw, 1),
            "how": "MFMA: register-only chains of 32x32x16 bf16 MFMAs over 2048 workgroups of 4 waves; "
                   "copy: torch copy of 1 GiB fp32 (bytes read + written)"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, weights, tok, tgt, normuon=False, windows=None):
    """Time the oracle on a bounded sample and scale it to one full step."""
    import oracle  # test infrastructure: used here only for the CPU baseline leg

    cores = len(os.sched_getaffinity(0))
    L, B, T = cfg["depth"], cfg["batch"], cfg["seq"]
    t0 = time.perf_counter()
    oracle.forward_backward(weights, tok[:1], tgt[:1],
                            windows=None if windows is None else [None if w < 0 else w for w in windows])
    t_seq = time.perf_counter() - t0
    names = [f"h0.{n}" for n in ("wq", "wk", "wv", "wo", "wfc", "wproj")]
    sub_w = {k: weights[k] for k in names}
    rng = np.random.default_rng(9)
    sub_g = {k: (rng.standard_normal(sub_w[k].shape, dtype=np.float32) * 1e-3) for k in names}
    sub_m = {k: np.zeros_like(v) for k, v in sub_w.items()}
    t0 = time.perf_counter()
    if normuon:
        sub_v = {k: np.zeros(max(v.shape), dtype=np.float32) for k, v in sub_w.items()}
        oracle.normuon_step(sub_w, sub_g, sub_m, sub_v, syn.MUON_LR, syn.MUON_MOMENTUM, NORMUON_BETA2,
                            syn.NS_COEFFS)
    else:
        oracle.muon_step(sub_w, sub_g, sub_m, syn.MUON_LR, syn.MUON_MOMENTUM, syn.NS_COEFFS)
    t_muon_layer = time.perf_counter() - t0
    ad_w = {k: weights[k] for k in ("wte", "lm_head")}
    ad_g = {k: (rng.standard_normal(v.shape, dtype=np.float32) * 1e-3) for k, v in ad_w.items()}
    ad_z = {k: np.zeros_like(v) for k, v in ad_w.items()}
    t0 = time.perf_counter()
    oracle.adamw_step(ad_w, ad_g, ad_z, ad_z, 1, ADAMW["lr"], ADAMW["beta1"], ADAMW["beta2"], ADAMW["eps"],
                      ADAMW["weight_decay"])
    t_adamw = time.perf_counter() - t0
    t_step = B * t_seq + L * t_muon_layer + t_adamw
    return {
        "value": round(B * T / t_step, 3),
        "unit": "tokens/s",
        "cores": cores,
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": (f"fp32 NumPy oracle: fwd+bwd of 1 of {B} sequences ({T} tokens, {t_seq:.2f} s), "
                   f"{'NorMuon' if normuon else 'Muon'} of 1 of {L} layers ({t_muon_layer:.2f} s) and AdamW of wte and lm_head "
                   f"({t_adamw:.2f} s), scaled to the full step (sequences and layers are "
                   f"independent units of equal cost)"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="d20", choices=sorted(syn.CONFIGS))
    ap.add_argument("--accum", type=int, default=1,
                    help="microbatches per optimizer step (gradient accumulation)")
    ap.add_argument("--window-pattern", default=None,
                    help="per-layer attention windows, e.g. SSSL (S: seq/2 keys, L: full causal)")
    ap.add_argument("--kv-heads", type=int, default=None,
                    help="key/value heads (grouped-query attention; default: every head)")
    ap.add_argument("--normuon", action="store_true",
                    help="NorMuon variance reduction after Newton-Schulz (normuon_step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak-probes", action="store_true",
                    help="skip the measured MFMA-rate and copy-bandwidth probes")
    ap.add_argument("--no-isolated-timings", action="store_true",
                    help="skip the separate AdamW / Muon timings after the timed steps (keeps a "
                         "kernel trace to whole steps)")
    ap.add_argument("--packed", action="store_true",
                    help="feed rows from the library's BOS best-fit packer over seeded synthetic "
                         "documents instead of independent Zipf rows")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="launch one plain device copy of this many MiB before the steps "
                         "(the calibration kernel for rocprofv3 FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU step only: the library has no multi-GPU path "
              "(each data-parallel rank would run this same step on its share of the batch). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from gpt_pretraining_step_bf16_amd.step import TrainState, window_pattern

    cfg = syn.CONFIGS[args.config]
    L, V, T, B = cfg["depth"], cfg["vocab"], cfg["seq"], cfg["batch"]
    dims = syn.model_dims(L)
    d = dims["d"]
    print(f"[bench] config {args.config}: depth {L} width {d} vocab {V} seq {T} batch {B}",
          file=sys.stderr, flush=True)
    weights = syn.init_weights(L, V, seed=0, kv_heads=args.kv_heads)
    packing = None
    if args.packed:
        # Rows of T + 1 tokens from the packer (host code in the library). The
        # buffer is settled for 20 batches first; the timed steps then run on
        # the next batch, resident in HBM like the Zipf rows.
        from gpt_pretraining_step_bf16_amd import binding

        doc_tok, doc_off = syn.synthetic_documents(max(4096, 40 * B * (T + 1) // 1000), V, seed=3)
        pk = binding.BestFitPacker(doc_tok, doc_off, syn.PACK_BUFFER_DOCS)
        t_pack = time.perf_counter()
        for _ in range(20):
            pk.pack(B, T + 1)
        t_pack = (time.perf_counter() - t_pack) / 20
        cut0 = pk.tokens_cut
        rows = pk.pack(B, T + 1)
        cut = pk.tokens_cut - cut0
        tok, tgt = syn.split_tokens(rows)
        packing = {"buffer_docs": syn.PACK_BUFFER_DOCS,
                   "doc_len": f"round(exp(N({syn.DOC_LEN_MU}, {syn.DOC_LEN_SIGMA}))) tokens, BOS first",
                   "tokens_cut_frac": round(cut / (B * (T + 1) + cut), 4),
                   "rows_start_with_bos": bool((rows[:, 0] == V - 1).all()),
                   "host_pack_ms_per_batch": round(t_pack * 1e3, 3)}
    else:
        tok, tgt = syn.split_tokens(syn.zipf_ids(B, T, V, seed=1))
    st = TrainState(L, V, T, B, kv_heads=args.kv_heads)
    st.load_weights(weights)
    windows = window_pattern(L, T, args.window_pattern) if args.window_pattern else None
    st.set_windows(windows)
    tok_d = torch.from_numpy(tok).cuda()
    tgt_d = torch.from_numpy(tgt).cuda()
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: {n * 4} bytes read and written", file=sys.stderr, flush=True)
        del src, dst

    accum = max(1, args.accum)
    opt_step = [0]

    def block_update():
        if args.normuon:
            st.normuon(syn.MUON_LR, syn.MUON_MOMENTUM, NORMUON_BETA2, syn.NS_COEFFS)
        else:
            st.muon(syn.MUON_LR, syn.MUON_MOMENTUM, syn.NS_COEFFS)

    def step():
        for i in range(accum):
            st.fwd_bwd(tok_d, tgt_d, accumulate=i > 0)
        block_update()
        opt_step[0] += 1
        st.adamw(ADAMW["lr"], ADAMW["beta1"], ADAMW["beta2"], ADAMW["eps"], ADAMW["weight_decay"],
                 opt_step[0])

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup step {i} loss {float(st.loss.item()):.5f}", file=sys.stderr, flush=True)
    if st.check() != 0:
        raise RuntimeError("device reported an out-of-range token")

    def timed(nsteps):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        for _ in range(nsteps):
            step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), time.perf_counter() - w0

    # Headline: the timed steps run with no per-launch events.
    elapsed_ms, wall = timed(args.steps)
    loss = float(st.loss.item())
    if not np.isfinite(loss):
        raise RuntimeError(f"non-finite loss {loss}")
    # Breakdown: a second timed pass of the same steps with HIP events around
    # every launch of the GEMM, attention and Newton-Schulz kernels, recorded
    # on the stream they run on.
    prof_steps = max(1, min(args.steps, 5))
    st.model.profile_enable(True)
    prof_ms, _ = timed(prof_steps)
    prof = {name: st.model.profile_read(cat) for name, cat in
            (("gemm", 0), ("attn_fwd", 1), ("attn_bwd", 2), ("ns_gemm", 3))}
    st.model.profile_enable(False)

    ms_step = elapsed_ms / args.steps
    tokens_per_s = accum * B * T * args.steps / (elapsed_ms / 1e3)
    dkv = 128 * st.model.kv_heads
    f_tok = flops_per_token(L, d, V, T, windows, dkv)
    mfu = tokens_per_s * f_tok / PEAK_BF16_FLOPS
    ns_alg = ns_flops(L, d, dkv=dkv)
    mfma_work = (tokens_per_s * f_tok + ns_alg / (ms_step / 1e3)) / PEAK_BF16_FLOPS
    adamw_ms = block_ms = fwd_bwd_ms = None
    if not args.no_isolated_timings:
        def iso(fn, n):
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record()
            for _ in range(n):
                fn()
            a1.record()
            torch.cuda.synchronize()
            return a0.elapsed_time(a1) / n

        def adamw_once():
            opt_step[0] += 1
            st.adamw(ADAMW["lr"], ADAMW["beta1"], ADAMW["beta2"], ADAMW["eps"], ADAMW["weight_decay"],
                     opt_step[0])

        # Each call alone, timed the same way (HIP events on the current stream).
        adamw_ms = iso(adamw_once, 5)
        block_ms = iso(block_update, 3)
        fwd_bwd_ms = iso(lambda: st.fwd_bwd(tok_d, tgt_d), 3)
    for name, (ms, fl, n) in prof.items():
        tf = fl / (ms / 1e3) / 1e12 if ms > 0 else 0.0
        extra = ""
        if name == "ns_gemm" and ms > 0:
            extra = f"  (executed; algorithmic {ns_alg * prof_steps / (ms / 1e3) / 1e12:.1f})"
        print(f"[bench] {name:9s} {ms / prof_steps:9.2f} ms/step  {n // prof_steps:5d} launches/step"
              f"  {tf:8.1f} TFLOP/s{extra}", file=sys.stderr, flush=True)
    g_ms, g_fl, g_n = prof["gemm"]
    # The head runs over token chunks of at most 1 GiB of bf16 logits (at least 256 rows).
    head_chunk = min(B * T, max(256, (1 << 30) // (2 * V)))
    g_bytes, g_launches = gemm_bytes_per_step(L, d, V, B * T, head_chunk, dkv)
    achieved = g_fl / (g_ms / 1e3) / 1e12 if g_ms > 0 else 0.0
    peaks = None if args.no_peak_probes else measured_peaks(torch)
    roofline = {
        "kernel": "gemm_pp_kernel + gemm_bf16_kernel (projection, head and weight-gradient GEMMs of fwd+bwd)",
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_FLOPS / 1e12,
        "unit": "TFLOP/s",
        "frac": round(achieved / (PEAK_BF16_FLOPS / 1e12), 4),
        "traffic": gemm_traffic(),
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "algorithmic_bytes_per_launch": round(g_bytes / g_launches),
        "launches_per_step": g_n // prof_steps,
        "ms_per_step": round(g_ms / prof_steps, 3),
        "timing": f"HIP events around each launch over a second timed pass of {prof_steps} steps",
    }
    if peaks:
        roofline["frac_of_measured_peak"] = round(achieved / peaks["mfma_bf16_tflops"], 4)
    ns_ms = prof["ns_gemm"][0] / prof_steps
    amort = None
    if fwd_bwd_ms is not None:
        # The single-GPU accumulation mode: 8 microbatches per optimizer step.
        t8 = fwd_bwd_ms + (block_ms + adamw_ms) / 8.0
        amort = round(B * T / (t8 / 1e3) * f_tok / PEAK_BF16_FLOPS, 4)
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic (seeded documents of Zipf(1.1) token ids, BOS best-fit packed; N(0, 0.02) weights)"
                 if packing else "synthetic (seeded Zipf(1.1) token ids, N(0, 0.02) weights)"),
        "config": {
            "workload": f"{args.config}: depth {L}, width {d}, {dims['heads']} heads x 128, MLP {4 * d}, "
                        f"vocab {V}, seq {T}, microbatch {B}"
                        + (f" x {accum} accumulated" if accum > 1 else "")
                        + (f"; attention windows {args.window_pattern.upper()} (S = {T // 2} keys)"
                           if args.window_pattern else "")
                        + (f"; {args.kv_heads} key/value heads" if args.kv_heads else "")
                        + "; fwd+bwd+" + ("NorMuon" if args.normuon else "Muon")
                        + " (5 Newton-Schulz steps)+AdamW (wte, lm_head)",
            "global_batch": accum * B,
            "seq_len": T,
            "parallelism": "none (1 GPU)",
            **({"packing": packing} if packing else {}),
        },
        "mfu": round(mfu, 4),
        "mfu_vs_measured_peak": None if not peaks else round(mfu * PEAK_BF16_FLOPS / 1e12
                                                             / peaks["mfma_bf16_tflops"], 4),
        "mfma_work_utilisation": round(mfma_work, 4),
        "mfu_amortised_8_microbatches": amort,
        "loss": round(loss, 5),
        "wall_s_timed": round(wall, 3),
        "ms_per_step_with_launch_events": round(prof_ms / prof_steps, 3),
        "fwd_bwd_ms": None if fwd_bwd_ms is None else round(fwd_bwd_ms, 3),
        "adamw_ms": None if adamw_ms is None else round(adamw_ms, 3),
        ("normuon_ms" if args.normuon else "muon_ms"): None if block_ms is None else round(block_ms, 3),
        "newton_schulz": {"ms_per_step": round(ns_ms, 3),
                          "algorithmic_tflops": round(ns_alg / (ns_ms / 1e3) / 1e12, 1) if ns_ms > 0 else None,
                          "executed_tflops": round(prof["ns_gemm"][1] / prof_steps / (ns_ms / 1e3) / 1e12, 1)
                          if ns_ms > 0 else None},
        "measured_peaks": peaks,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, weights, tok, tgt, args.normuon, windows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
