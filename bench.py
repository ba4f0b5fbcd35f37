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
    ap.add_argument("--calibrate-mfma", choices=("bf16", "int8"), default=None,
                    help="only run the matrix-core probe (dense MFMA rate at the running clock)")
    ap.add_argument("--membound", action="store_true",
                    help="only time the memory-bound kernels one by one at the workload's sizes")
    ap.add_argument("--vendor-gemm", default=None, metavar="M,N,K",
                    help="only time one bf16 product of this shape with h3_gemm_bf16 and with "
                         "PyTorch's F.linear (the vendor library), for comparison")
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


def calibrate_mfma(kind: str):
    """Times the matrix-core probe: two workgroups of four waves per CU, each wave issuing
    rounds of eight independent 32x32 MFMAs with no memory traffic.  Prints the sustained rate
    and the clock it implies (1024 bf16 FLOP, or 2048 int8 OP, per SIMD per cycle)."""
    import torch
    from video_diffusion_transformer_fwd_amd import binding as B
    int8 = kind == "int8"
    wgs, iters = 512, 40000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    B.h3_mfma_probe(int8, 100, wgs, out)
    torch.cuda.synchronize()
    per_instr = 65536.0 if int8 else 32768.0
    ops = wgs * 4 * iters * 8 * per_instr
    res = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.h3_mfma_probe(int8, iters, wgs, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        res.append(ms)
    ms = sorted(res)[len(res) // 2]
    rate = ops / (ms * 1e-3) / 1e12
    simds, per_clk = 1024, (2048.0 if int8 else 1024.0)
    print(json.dumps({"calibrate_mfma": kind, "ms": round(ms, 3), "ops_per_launch": ops,
                      "rate_tops": round(rate, 1), "peak_spec_tops": PEAK_INT8_TOPS if int8 else PEAK_BF16_TFLOPS,
                      "implied_clock_ghz": round(rate * 1e12 / (simds * per_clk) / 1e9, 3)}))


def membound(w):
    """The memory-bound kernels of the path, one at a time at the workload's sizes, through the
    op-level entry points: median of 5 launches (HIP events), algorithmic bytes / time.  Inputs
    are random device tensors; a plain device copy of the residual stream's size is the
    reference rate."""
    import torch
    from video_diffusion_transformer_fwd_amd import binding as B
    from video_diffusion_transformer_fwd_amd.runtime import Geometry
    geo = Geometry(w)
    n, d, F, C, D = geo.n_tokens, w.d_model, w.ffn_dim, w.latent_ch, w.head_dim
    dev = "cuda"
    bf = lambda *shape: torch.randn(*shape, device=dev).to(torch.bfloat16)
    f32 = lambda *shape, s=0.2: torch.randn(*shape, device=dev) * s
    x, y, xo, nn_ = bf(n, d), bf(n, d), bf(n, d), torch.empty(n, d, dtype=torch.bfloat16, device=dev)
    gate, sh, sc = f32(d), f32(d), f32(d)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    out = []

    def report(name, ms, nbytes):
        rec = {"kernel": name, "us": round(ms * 1e3, 1), "bytes": int(nbytes),
               "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "frac_of_8tb": round(nbytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)}
        out.append(rec)
        print(json.dumps(rec), flush=True)

    src = bf(n, d)
    dst = torch.empty_like(src)
    report("device copy (torch copy_) of [N, d] bf16", timed(lambda: dst.copy_(src)), 4 * n * d)
    report("gate_adaln fused: x' = x + g y, AdaLN(x')",
           timed(lambda: B.h3_gate_adaln(x, y, gate, xo, sh, sc, nn_)), 8 * n * d)
    report("adaln", timed(lambda: B.h3_gate_adaln(x, None, None, None, sh, sc, nn_)), 4 * n * d)
    report("gate only", timed(lambda: B.h3_gate_adaln(x, y, gate, xo, None, None, None)), 6 * n * d)
    h = bf(n, F)
    q8 = torch.empty(n, F, dtype=torch.int8, device=dev)
    s_row = torch.empty(n, 1, dtype=torch.float32, device=dev)
    report("quant_rows (row scale) of the FC2 input [N, F]",
           timed(lambda: B.h3_quant_rows(h, q8, s_row, F)), 3 * n * F + 4 * n)
    s_grp = torch.empty(n, F // 1024, dtype=torch.float32, device=dev)
    report("quant_rows (1024-channel groups) of [N, F]",
           timed(lambda: B.h3_quant_rows(h, q8, s_grp, 1024)), 3 * n * F + 4 * n * (F // 1024))
    del h, q8
    qkvq = bf(n, 4 * d)
    table = torch.empty(n, D // 2, 2, dtype=torch.float32, device=dev)
    B.h3_rope_table(geo.geom, D, table)
    gq = (1 + 0.02 * torch.randn(D, device=dev)).to(torch.bfloat16)
    gk = (1 + 0.02 * torch.randn(D, device=dev)).to(torch.bfloat16)
    report("qk_norm_rope (unfused) on the q, k columns of [N, 4d]",
           timed(lambda: B.h3_qk_norm_rope(qkvq, n, d, D, gq, gk, True, table)),
           8 * n * d + n * (D // 2) * 8)
    del qkvq
    nr = geo.f_lat * geo.grid_h * ((geo.grid_w + 1) // 2)
    xr = torch.empty(nr, d, dtype=torch.bfloat16, device=dev)
    report("token merge [N, d] -> [N_r, d]", timed(lambda: B.h3_token_reduce(0, geo.geom, d, x, None, xr)),
           2 * n * d + 2 * nr * d)
    xs = x.clone()
    report("token restore (bypass, in place)", timed(lambda: B.h3_token_reduce(1, geo.geom, d, xr, xs, xs)),
           2 * nr * d + 4 * n * d)
    lat, vel = f32(n, C, s=1.0), f32(n, C, s=1.0)
    report("euler step [N, C] float32", timed(lambda: B.h3_euler_step(lat, vel, 0.75, 0.5)), 12 * n * C)
    print(json.dumps({"membound": w.name, "tokens": n, "d_model": d, "ffn": F, "kernels": out}))


def vendor_gemm(shape: str):
    """One product C = A W^T + b ([M, K] x [N, K]) by h3_gemm_bf16 and by torch F.linear (which
    dispatches to the vendor GEMM library on this platform): median of 5 launches each."""
    import torch
    import torch.nn.functional as F
    from video_diffusion_transformer_fwd_amd import binding as B
    M, N, K = (int(v) for v in shape.split(","))
    A = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    W = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
    b = (torch.randn(N, device="cuda") * 0.02).to(torch.bfloat16)
    C = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    res = {}
    for name, fn in (("h3_gemm_bf16", lambda: B.h3_gemm_bf16(A, W, C, bias=b)),
                     ("torch F.linear", lambda: F.linear(A, W, b))):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[2]
        res[name] = {"ms": round(ms, 4), "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
    print(json.dumps({"vendor_gemm": [M, N, K], **res}))


def traffic_for(kernel_src: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if taken on this source and
    this workload."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = open(os.path.join(ROOT, "video_diffusion_transformer_fwd_amd", "csrc", kernel_src), "rb").read()
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest() or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float):
    """Oracle (float64 NumPy) on a bounded sample: the first blocks of one fresh evaluation,
    in order, until about ``budget_s`` seconds of oracle time are spent.  Geometry and active
    list come from the oracle's own host logic."""
    import threadpoolctl
    from oracle import dit, host
    from video_diffusion_transformer_fwd_amd import synthetic as S

    f_lat = host.latent_frames(host.align_frames(w.frames))
    gh, gw, scale = host.token_grid(w.width, w.height)
    n = host.n_tokens(f_lat, gh, gw)
    to64 = lambda t: t.to("cpu").double().numpy()
    g = {k: to64(v) for k, v in S.global_weights(w).items()}
    active = host.select_layers(g["mod_table"], w.n_active)
    ctx = to64(S.context(w))
    mod, _ = dit.modulation(g, 1.0)
    coords = dit.rope_coords(f_lat, gh, gw, scale)
    x = dit.patch_embed(to64(S.latent(w, n)), g)
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    done, t_used = 0, 0.0
    while done < len(active):
        b = active[done]
        blk = {k: to64(v) for k, v in S.block_weights(w, b).items()}
        t0 = time.perf_counter()
        x = dit.block_forward(x, blk, mod[b], ctx, coords, w.n_heads, fc2_mode=w.fc2_mode,
                              int8_linear=w.int8_linear)
        t_used += time.perf_counter() - t0
        done += 1
        if t_used >= budget_s:
            break
    return {"value": round(n * done / t_used, 1), "unit": "tokens·blocks/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"sampled, not the full loop: {done} of the {len(active)} active blocks of "
                      f"one fresh evaluation at {w.name} ({n} full-resolution tokens, sigma 1), "
                      f"float64 NumPy oracle, {t_used:.1f} s of oracle time"}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.calibrate_mfma:
        calibrate_mfma(args.calibrate_mfma)
        return
    if args.vendor_gemm:
        vendor_gemm(args.vendor_gemm)
        return
    if args.membound:
        from video_diffusion_transformer_fwd_amd import synthetic as S
        membound(S.WORKLOADS[args.workload])
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
    # algorithmic operations of the timed forwards, split by the matrix-core type each product
    # runs on: QKV + cross Q (2 r d 4d), attention (4 r^2 d + 4 r L d), output projections
    # (4 r d^2), FC1 (2 r d F), FC2 (2 r F d)
    d_, L_, F_ = w.d_model, w.ctx_len, w.ffn_dim
    ops = {"bf16": 0.0, "int8": 0.0}
    for r in timed_rows:
        ops["int8" if w.int8_linear else "bf16"] += 2.0 * r * d_ * 4 * d_ + 2.0 * r * d_ * F_
        ops["bf16"] += 4.0 * r * r * d_ + 4.0 * r * L_ * d_ + 4.0 * r * d_ * d_
        ops["int8" if w.fc2_mode != "bf16" else "bf16"] += 2.0 * r * F_ * d_
    # time-weighted fraction of the matrix-core peaks: each product's operations over its own
    # type's peak, summed, over the elapsed time
    mfma_frac = (ops["bf16"] / PEAK_BF16_TFLOPS + ops["int8"] / PEAK_INT8_TOPS) / 1e12 / elapsed
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
        "mfma_frac_forward": round(mfma_frac, 4),
        "forward_ops": {"bf16_tflop": round(ops["bf16"] / 1e12, 3),
                        "int8_top": round(ops["int8"] / 1e12, 3),
                        "bf16_tflops": round(ops["bf16"] / 1e12 / elapsed, 1),
                        "int8_tops": round(ops["int8"] / 1e12 / elapsed, 1)},
        "roofline": {"bound": "mfma",
                     "kernel": ("fc1_gemm (int8 GEMM + dequant + GELU epilogue)" if w.int8_linear
                                else "fc1_gemm (bf16 GEMM + GELU epilogue)"),
                     "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TOP/s" if w.int8_linear else "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "flops_per_launch": fc1_flops, "avg_launch_ms": round(fc1_avg_ms, 5),
                     "launches": fc1_launches,
                     "traffic": None if w.int8_linear else traffic_for("k_gemm.hip", w.name)},
    }
    if not args.no_cpu:
        del model
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
