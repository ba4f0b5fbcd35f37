"""Benchmark of the DiT denoiser hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 512sq_22f] [--no-cpu]

One step = one denoise transition of the --steps 4 --reuse 1 schedule at 512x512x22 frames
(1536 tokens, 50 blocks): a fresh DiT evaluation (modulation, patch, 50 blocks, final
AdaLN + head) followed by the Euler update; steps walk the 4-step sigma grid cyclically.
The model (bf16 weights, 15 GB) and the latent are resident in HBM before timing starts.

Prints one JSON line: tokens*blocks/s over the K timed steps (nominal: N x active blocks per
fresh evaluation; with token pairing the actual count, sum of each block's own token count,
is reported beside it), ms per denoise step, the roofline of the dominant kernel (FC1 GEMM: its
launches are timed with HIP events on the launch stream during the timed steps; its algorithmic
FLOPs per launch = 2 N_b d F at the block's token count N_b), and the oracle's throughput on a
bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="512sq_22f")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times), the "
                         "reference for scaling HBM byte counters")
    return ap.parse_args()


def calibrate_copy(mib: int):
    """A plain copy of known size: counters taken on it scale FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.empty(mib * 2 ** 20, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": mib * 2 ** 20, "copies": 5}))


def traffic_for(kernel_src: str):
    """HBM bytes per launch from the committed counter summary, if taken on this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = open(os.path.join(ROOT, "video_diffusion_transformer_fwd_amd", "csrc", kernel_src), "rb").read()
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, budget_s: float):
    """Oracle (float64 NumPy) on a bounded sample: whole blocks of one fresh evaluation."""
    import numpy as np
    import threadpoolctl
    from oracle import dit
    from video_diffusion_transformer_fwd_amd import synthetic as S
    from video_diffusion_transformer_fwd_amd.runtime import Geometry

    geo = Geometry(w)
    to64 = lambda t: t.to("cpu").double().numpy()
    g = {k: to64(v) for k, v in S.global_weights(w).items()}
    ctx = to64(S.context(w))
    mod, _ = dit.modulation(g, 1.0)
    coords = dit.rope_coords(geo.f_lat, geo.grid_h, geo.grid_w, geo.scale)
    x = dit.patch_embed(to64(S.latent(w, geo.n_tokens)), g)
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    done, t_used = 0, 0.0
    while done < w.n_blocks:
        blk = {k: to64(v) for k, v in S.block_weights(w, done).items()}
        t0 = time.perf_counter()
        x = dit.block_forward(x, blk, mod[done], ctx, coords, w.n_heads)
        t_used += time.perf_counter() - t0
        done += 1
        if t_used >= budget_s:
            break
    return {"value": geo.n_tokens * done / t_used, "unit": "tokens*blocks/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of the {w.n_blocks} blocks of one fresh evaluation at "
                      f"{w.name} ({geo.n_tokens} tokens), float64 NumPy, {t_used:.1f} s"}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "runs on one GPU only: --gpus N > 1 is not supported (the "
                                   "multi-GPU sequence split is designed, not implemented)"}))
        sys.exit(2)
    import torch
    from video_diffusion_transformer_fwd_amd import binding as B
    from video_diffusion_transformer_fwd_amd import synthetic as S
    from video_diffusion_transformer_fwd_amd.runtime import DiTModel

    w = S.WORKLOADS[args.workload]
    t0 = time.time()
    model = DiTModel(w)
    print(f"# model resident in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    geo = model.geo
    n, nb_act = geo.n_tokens, w.n_active
    active = model.active()
    opts = model.opts()
    sig, fresh, n_fresh = B.h3_schedule(w.steps, w.reuse, w.core_reuse)
    # core-residual reuse: every step runs the patch and the head; the marked steps the core
    core_delta = (torch.empty((n, w.d_model), dtype=torch.float32, device=model.device)
                  if w.core_reuse > 1 else None)
    lat = model.initial_latent()
    v = torch.empty((n, w.latent_ch), dtype=torch.float32, device=model.device)
    ev_count = [0]

    def rows_per_block(eval_index):
        """Token count each active position runs at in this evaluation (token pairing shrinks the
        positions from merge_after up to restore_before - 2 to the reduced count)."""
        if not w.token_reduction:
            return [n] * nb_act
        plan = B.h3_token_plan(geo.f_lat, geo.grid_h, geo.grid_w, eval_index, nb_act, with_pairs=False)
        lo, hi = plan["merge_after"], plan["restore_before"] - 1
        return [plan["n_reduced"] if lo <= pos < hi else n for pos in range(nb_act)]

    timed_rows = []

    def step(k, timed=False):
        i = k % w.steps
        if core_delta is not None:
            e = ev_count[0] % max(n_fresh, 1)
            model.forward_cached(lat, float(sig[i]), bool(fresh[i]), core_delta, active, e, opts, v)
            if fresh[i]:
                ev_count[0] += 1
                if timed:
                    timed_rows.extend(rows_per_block(e))
        elif fresh[i]:
            e = ev_count[0] % max(n_fresh, 1)
            model.forward(lat, float(sig[i]), active, e, opts, v)
            ev_count[0] += 1
            if timed:
                timed_rows.extend(rows_per_block(e))
        B.h3_euler_step(lat, v, float(sig[i]), float(sig[i + 1]))

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    fresh_before = ev_count[0]
    B.h3_profile_begin(["fc1_gemm"], max_launches=args.steps * nb_act + 16)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.warmup, args.warmup + args.steps):
        step(k, timed=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    prof = B.h3_profile_end()
    n_evals = ev_count[0] - fresh_before

    ms_per_step = elapsed * 1e3 / args.steps
    tok_blocks = n * nb_act * n_evals / elapsed
    fc1_ms, fc1_launches = prof.get("fc1_gemm", (0.0, 0))
    fc1_avg_ms = fc1_ms / max(fc1_launches, 1)
    # algorithmic FLOPs of the timed FC1 launches: 2 N_b d F per block at its own token count
    fc1_flops_total = sum(2.0 * r * w.d_model * w.ffn_dim for r in timed_rows)
    fc1_flops = fc1_flops_total / max(fc1_launches, 1)
    achieved = fc1_flops_total / (fc1_ms * 1e-3) / 1e12 if fc1_launches else 0.0
    d_, L_, F_ = w.d_model, w.ctx_len, w.ffn_dim
    fwd_flops_total = sum(2 * r * d_ * 4 * d_ + 4 * r * r * d_ + 4 * r * L_ * d_ + 4 * r * d_ * d_
                          + 4 * r * d_ * F_ for r in timed_rows)
    actual_tok_blocks = sum(timed_rows) / elapsed
    peak = PEAK_INT8_TOPS if w.int8_linear else PEAK_BF16_TFLOPS
    out = {
        "metric": "DiT denoise-step ms & tokens·blocks/s at 512²×22f; % bf16 MFMA peak",
        "value": round(tok_blocks, 1),
        "unit": "tokens·blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+int8" if (w.int8_linear or w.fc2_mode != "bf16") else "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) latent)",
        "config": {"workload": w.name, "width": w.width, "height": w.height, "frames": w.frames,
                   "tokens": n, "blocks": nb_act, "d_model": w.d_model, "heads": w.n_heads,
                   "ffn": w.ffn_dim, "ctx_len": w.ctx_len, "steps": w.steps, "reuse": w.reuse,
                   "core_reuse": w.core_reuse, "fc2": w.fc2_mode, "int8_qkv_fc1": w.int8_linear,
                   "token_reduction": w.token_reduction},
        "ms_per_fresh_eval": round(elapsed * 1e3 / max(n_evals, 1), 3),
        "actual_tokens_blocks_per_s": round(actual_tok_blocks, 1),
        "mfma_frac_forward": round(fwd_flops_total / elapsed / 1e12 / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma",
                     "kernel": ("fc1_gemm (int8 GEMM + dequant + GELU epilogue)" if w.int8_linear
                                else "fc1_gemm (bf16 GEMM + GELU epilogue)"),
                     "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TOP/s" if w.int8_linear else "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "flops_per_launch": fc1_flops, "avg_launch_ms": round(fc1_avg_ms, 5),
                     "launches": fc1_launches,
                     "traffic": None if w.int8_linear else traffic_for("k_gemm.hip")},
    }
    if not args.no_cpu:
        del model
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
