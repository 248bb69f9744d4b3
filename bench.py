"""Throughput of one training step (forward + loss + backward) of the
depth-20 dense GPT on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload C4] [--no-cpu-baseline]
    python bench.py --decode-only --steps 256   # KV-cache prefill + decoding steps only
    python bench.py --kernel-only      # 3 launches of the roofline kernel + a 1 GiB copy
                                       # (for hardware-counter passes)

Prints one JSON line: tokens/s for the whole step (inputs resident in HBM),
milliseconds per step, MFU against the dense bf16 matrix-core peak, the
roofline of the dominant kernel (timed live with HIP events on the stream it
runs on) and the fp64 CPU oracle timed on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/sec and MFU, depth-20 fwd+bwd step on 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0           # MI355X dense bf16 matrix cores
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

WORKLOAD_NAMES = {
    "C1": "tiny GPT fwd+bwd fp32: depth 2, d 128, V 512, T 64, B 2",
    "C2": "small GPT fwd+bwd bf16: depth 4, d 256, V 8192, T 512, B 8",
    "C3": "mid GPT fwd+bwd bf16: depth 12, d 768, V 65536, T 2048, B 8",
    "C4": "speedrun-shape GPT fwd+bwd bf16: depth 20, d 1280, 10 heads, 1 KV head, "
          "V 65536, T 2048, B 32 (65,536 tokens/step)",
    "C5": "GPT-2-grade GPT fwd+bwd bf16: depth 26, d 1664, V 65536, T 2048, B 16",
}


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C4", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-all", action="store_true",
                    help="time only the fp64 oracle on every workload (no GPU)")
    ap.add_argument("--no-optimizer", action="store_true",
                    help="skip the separate timing of the optimizer step")
    ap.add_argument("--optimizer-only", action="store_true",
                    help="time only optimizer steps on a seeded synthetic gradient (for traces)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only KV-cache inference: a 1024-token prefill, then decoding steps")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the separate timing of KV-cache decoding")
    ap.add_argument("--no-eval", action="store_true",
                    help="skip the separate timing of the bits-per-byte evaluation")
    ap.add_argument("--lm-chunk-rows", type=int, default=0,
                    help="rows of the lm_head / loss chunk (0: the library default)")
    ap.add_argument("--kernel-only", action="store_true",
                    help="launch only the roofline kernel (3x) and a 1 GiB device copy (3x)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_mlp_up_c4_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "dense_gpt_pretraining_nanochat_amd", "csrc", "k_gemm.hip")


def measured_traffic(shape):
    """HBM bytes per launch of the roofline kernel from the stored counter
    passes (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads
    for a copy of known size), or None when the kernel source has changed
    since the counters were taken or the shape differs."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(GEMM_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != sha or list(t.get("shape", [])) != list(shape):
        return None
    return int(t["fetch_bytes"] + t["write_bytes"])


def roofline_after_steps(cfg, nc, torch, step, tok_d, tgt_d, reps=5):
    """The roofline kernel under the step's conditions (clocks, caches): one
    launch timed right after each of `reps` training steps, HIP events on the
    stream it is launched on."""
    M = cfg.batch * cfg.seq_len
    d = 64 * cfg.depth
    F = 4 * d
    et = torch.bfloat16 if cfg.dtype == nc.NC_BF16 else torch.float32
    A = torch.randn(M, d, device="cuda").to(et)
    B = (torch.randn(F, d, device="cuda") * 0.02).to(et)
    U = torch.empty(M, F, device="cuda", dtype=et)
    s = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        step.forward_backward(tok_d, tgt_d)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        nc.nc_op_gemm(cfg.dtype, 1, 1, nc.EPI_RELU2, A, B, U, None, M, F, d, d, d, F, stream=s)
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
    del A, B, U
    sec = sum(times) / len(times)
    ach = 2.0 * M * F * d / sec / 1e12
    return {"avg_us": round(sec * 1e6, 2), "achieved": round(ach, 2),
            "frac": round(ach / PEAK_BF16_TFLOPS, 4), "launches": reps,
            "how": "one launch timed right after each training step (the step's clocks and caches)"}


def dominant_kernel_roofline(cfg, nc, torch, reps=20, warm=25):
    """Times the MLP up-projection GEMM (tokens x 4d x d, relu^2 epilogue;
    the largest single contraction of the step) on its own, with HIP events
    on the stream it is launched on. A burst of this kernel right after the
    step runs slower for its first ~15 launches while the clocks settle, so
    `warm` untimed launches come first."""
    M = cfg.batch * cfg.seq_len
    d = 64 * cfg.depth
    F = 4 * d
    bf = cfg.dtype == nc.NC_BF16
    et = torch.bfloat16 if bf else torch.float32
    A = torch.randn(M, d, device="cuda").to(et)
    B = (torch.randn(F, d, device="cuda") * 0.02).to(et)
    U = torch.empty(M, F, device="cuda", dtype=et)
    s = torch.cuda.current_stream()
    for _ in range(warm):
        nc.nc_op_gemm(cfg.dtype, 1, 1, nc.EPI_RELU2, A, B, U, None, M, F, d, d, d, F, stream=s)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(s)
    for _ in range(reps):
        nc.nc_op_gemm(cfg.dtype, 1, 1, nc.EPI_RELU2, A, B, U, None, M, F, d, d, d, F, stream=s)
    ev1.record(s)
    ev1.synchronize()
    sec = ev0.elapsed_time(ev1) / 1e3 / reps
    flops = 2.0 * M * F * d
    peak = PEAK_BF16_TFLOPS if bf else PEAK_F32_TFLOPS
    ach = flops / sec / 1e12
    del A, B, U
    return {"kernel": "gemm_bf16_kernel<Relu2, A k-contiguous, B k-contiguous> "
                      "(MLP up-projection, forward)",
            "shape": [M, F, d], "bound": "mfma", "achieved": round(ach, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(ach / peak, 4), "avg_us": round(sec * 1e6, 2),
            "flops_per_launch": flops, "warmup_launches": warm, "timed_launches": reps,
            "traffic": measured_traffic([M, F, d])}


def ns_flops(c):
    """Matrix-core FLOPs of Muon's Newton-Schulz iterations for one optimizer
    step: per matrix [R, C] with r = min, c = max, each iteration is
    X X^T (2 r r c), A A^T (2 r^3) and B X (2 r r c)."""
    d = 64 * c.depth
    mats = [(d + 256, d), (d, d), (4 * d, d), (d, 4 * d)]
    per_layer = sum(4 * min(R, C) ** 2 * max(R, C) + 2 * min(R, C) ** 3 for R, C in mats)
    return 5 * c.depth * per_layer


def optimizer_timing(step, nc, torch, c, reps=5):
    """One optimizer step (global-norm clip, AdamW on E and U, Muon with 5
    Newton-Schulz iterations on every block matrix) on the step's gradient,
    timed with HIP events on the stream it runs on."""
    o = nc.nc_optim_config(0.004, 0.8, 0.95, 1e-10, 0.0, 0.02, 0.95, 0.0, 1.0, 5, 1)
    s = torch.cuda.current_stream()
    saved = step.params.clone()
    for k in range(2):
        o.step = k + 1
        step.optimizer_step(o)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(s)
    for k in range(reps):
        o.step = k + 3
        step.optimizer_step(o)
    ev1.record(s)
    ev1.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    step.params.copy_(saved)
    fl = ns_flops(c)
    return {"ms_per_step": round(ms, 3), "newton_schulz_flops": fl,
            "newton_schulz_tflops_if_all_time": round(fl / (ms / 1e3) / 1e12, 1),
            "state_bytes": int(step.opt_state.numel() * 4),
            "what": "clip + AdamW(E, U) + Muon(5 Newton-Schulz steps) over all 502M parameters; "
                    "not part of the timed training step"}


def bpb_timing(step, nc, torch, c, tok_d, tgt_d, reps=3):
    """Bits-per-byte evaluation of the step's batch (the forward pass, the loss
    and an fp64 byte-weighted reduction) with a synthetic byte table."""
    from dense_gpt_pretraining_nanochat_amd import inputs
    tb = torch.from_numpy(inputs.make_token_bytes(c.vocab_size, 7)).cuda()
    s = torch.cuda.current_stream()
    step.eval_bpb(tok_d, tgt_d, tb)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(s)
    for _ in range(reps):
        r = step.eval_bpb(tok_d, tgt_d, tb)
    ev1.record(s)
    ev1.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    v = r.cpu().tolist()
    return {"ms_per_batch": round(ms, 3), "tokens_per_s": round(c.batch * c.seq_len / (ms / 1e3), 1),
            "bits_per_byte": v[2], "bytes": int(v[1]),
            "what": "forward + loss + byte-weighted fp64 reduction over the timed batch "
                    "(synthetic byte table); not part of the timed training step"}


def decode_bytes(c, pos):
    """Algorithmic HBM bytes of one decoding step at position pos: every block
    matrix and the lm_head read once, the batch's embedding rows, the cached
    k-hat and v of positions 0..pos read and position pos written, per layer
    and sequence (bf16)."""
    d = 64 * c.depth
    esz = 2 if c.dtype == "bf16" else 4
    block = (d + 256) * d + d * d + 2 * 4 * d * d
    weights = (c.depth * block + c.vocab_size * d) * esz
    kv = c.depth * c.batch * (pos + 2) * 256 * esz
    return weights + c.batch * d * esz + kv + c.batch * c.vocab_size * 4


def decode_timing(nc, torch, c, params, T0=1024, nsteps=128):
    """Prefill T0 tokens of every sequence, then `nsteps` decoding steps,
    each timed as a whole with HIP events on the stream they run on."""
    import numpy as np

    from dense_gpt_pretraining_nanochat_amd import inputs
    cfg = nc.nc_config_from_depth(c.depth, c.vocab_size, c.seq_len, c.batch, c.dtype)
    max_seq = T0 + nsteps + 8
    dec = nc.Decoder(cfg, params, max_seq)
    tok, _ = inputs.make_tokens(c.vocab_size, T0 + nsteps + 8, c.batch, 4321, "zipf")
    prompt = torch.from_numpy(np.ascontiguousarray(tok[:, :T0])).cuda()
    cols = [torch.from_numpy(np.ascontiguousarray(tok[:, p])).cuda() for p in range(tok.shape[1])]
    s = torch.cuda.current_stream()
    dec.prefill(prompt)                                  # warm
    for p in range(T0, T0 + 4):
        dec.step(cols[p])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record(s)
    dec.prefill(prompt)
    ev[1].record(s)
    for p in range(T0, T0 + nsteps):
        dec.step(cols[p])
    ev[2].record(s)
    ev[2].synchronize()
    pre_ms = ev[0].elapsed_time(ev[1])
    dec_ms = ev[1].elapsed_time(ev[2]) / nsteps
    status = dec.status()
    by = sum(decode_bytes(c, p) for p in range(T0, T0 + nsteps)) / nsteps
    return {"batch": c.batch, "prompt_tokens": T0, "decode_steps": nsteps,
            "positions": [T0, T0 + nsteps - 1],
            "prefill_ms": round(pre_ms, 3),
            "prefill_tokens_per_s": round(c.batch * T0 / (pre_ms / 1e3), 1),
            "decode_ms_per_step": round(dec_ms, 4),
            "decode_tokens_per_s": round(c.batch / (dec_ms / 1e3), 1),
            "decode_algorithmic_bytes_per_step": int(by),
            "decode_hbm_frac": round(by / (dec_ms / 1e3) / (PEAK_HBM_GBS * 1e9), 4),
            "device_status": status,
            "what": "KV-cache inference at the training shape (bf16, cache of the whole "
                    "context); not part of the timed training step"}


def decode_only(a):
    import torch

    import dense_gpt_pretraining_nanochat_amd as nc
    from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS
    c = PRESETS[a.workload]
    cfg = nc.nc_config_from_depth(c.depth, c.vocab_size, c.seq_len, c.batch, c.dtype)
    pdt = torch.bfloat16 if cfg.dtype == nc.NC_BF16 else torch.float32
    params = torch.zeros(nc.nc_param_count(cfg), dtype=pdt, device="cuda")
    nc.nc_init_params(SEEDS[a.workload][0], cfg, params)
    t = decode_timing(nc, torch, c, params, T0=min(1024, c.seq_len), nsteps=a.steps)
    print(json.dumps({"decode_only": a.workload, **t}), flush=True)


def optimizer_only(a):
    """Optimizer steps alone at the workload's shape: parameters from
    nc_init_params, a seeded normal gradient, 2 untimed + --steps timed."""
    import torch

    import dense_gpt_pretraining_nanochat_amd as nc
    from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS
    c = PRESETS[a.workload]
    cfg = nc.nc_config_from_depth(c.depth, c.vocab_size, c.seq_len, c.batch, c.dtype)
    step = nc.Step(cfg)
    step.init(SEEDS[a.workload][0])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    step.grads.normal_(0.0, 1e-3, generator=gen)
    t = optimizer_timing(step, nc, torch, c, reps=a.steps)
    print(json.dumps({"optimizer_only": a.workload, **t}), flush=True)


def kernel_only(a):
    """Three launches of the roofline kernel at the workload's shape, then three
    1 GiB device-to-device copies (the counter calibration), nothing else."""
    import torch

    import dense_gpt_pretraining_nanochat_amd as nc
    from dense_gpt_pretraining_nanochat_amd.config import PRESETS
    c = PRESETS[a.workload]
    cfg = nc.nc_config_from_depth(c.depth, c.vocab_size, c.seq_len, c.batch, c.dtype)
    M, d = c.batch * c.seq_len, 64 * c.depth
    F = 4 * d
    et = torch.bfloat16 if cfg.dtype == nc.NC_BF16 else torch.float32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    A = torch.randn(M, d, device="cuda", generator=gen).to(et)
    B = (torch.randn(F, d, device="cuda", generator=gen) * 0.02).to(et)
    U = torch.empty(M, F, device="cuda", dtype=et)
    for _ in range(3):
        nc.nc_op_gemm(cfg.dtype, 1, 1, nc.EPI_RELU2, A, B, U, None, M, F, d, d, d, F)
    src = torch.ones(256 * 1024 * 1024, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"kernel_only": a.workload, "gemm_shape": [M, F, d],
                      "copy_bytes": src.numel() * 4}), flush=True)


def host_facts():
    """The host the oracle runs on: usable cores, CPU model, BLAS library."""
    from threadpoolctl import threadpool_info
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    b = blas[0] if blas else {}
    return {"host_cores": cores, "cpu_model": model,
            "blas": f"{b.get('internal_api', 'unknown')} {b.get('version', '')}".strip(),
            "blas_threads": int(b.get("num_threads", 1))}


def oracle_timing(workload, rows):
    """The fp64 oracle (as it stands) forward + loss + backward on whole rows
    of the workload's batch (same seeded params and tokens as the GPU run):
    seconds and tokens/s on this host."""
    import oracle
    from dense_gpt_pretraining_nanochat_amd import inputs
    from dense_gpt_pretraining_nanochat_amd.config import PRESETS, SEEDS, TOKEN_LAW
    c = PRESETS[workload]
    pseed, dseed = SEEDS[workload]
    ocfg = oracle.OracleConfig(depth=c.depth, vocab=c.vocab_size, seq_len=c.seq_len, batch=c.batch)
    flat = inputs.make_params(oracle.layout(ocfg), oracle.param_count(ocfg, padded=True), pseed,
                              c.dtype, c.depth)
    p64 = inputs.as_float64(flat, c.dtype)
    del flat
    tok, tgt = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, TOKEN_LAW[workload])
    t0 = time.perf_counter()
    oracle.forward_backward(ocfg, p64, tok, tgt, rows=list(range(rows)), M=c.batch * c.seq_len)
    dt = time.perf_counter() - t0
    ntok = rows * c.seq_len
    return {"workload": workload, "rows": rows, "tokens": ntok, "seconds": round(dt, 2),
            "tokens_per_s": round(ntok / dt, 3)}


def cpu_baseline(workload):
    """One full row (all seq_len tokens) of the benched workload through the
    oracle, with the host facts."""
    t = oracle_timing(workload, 1)
    h = host_facts()
    return {"value": t["tokens_per_s"], "unit": "tokens/s", "cores": h["blas_threads"],
            "kind": "oracle", "seconds": t["seconds"],
            "sample": f"{workload}: batch row 0, all {t['tokens']} tokens, fp64 forward + loss + "
                      f"backward (the oracle as it stands)", **h}


def cpu_baseline_all():
    """The oracle on every workload: the two small ones on their whole batch,
    the three large ones on one full row each."""
    from dense_gpt_pretraining_nanochat_amd.config import PRESETS
    out = []
    for w in ("C1", "C2", "C3", "C4", "C5"):
        rows = PRESETS[w].batch if w in ("C1", "C2") else 1
        out.append(oracle_timing(w, rows))
        print(json.dumps({"progress": out[-1]}), flush=True)
    print(json.dumps({"cpu_baseline_all": out, **host_facts()}), flush=True)


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the step runs on a single GPU; see the sharding notes)", file=sys.stderr)
        sys.exit(2)
    if a.cpu_baseline_all:
        cpu_baseline_all()
        return
    if a.kernel_only:
        kernel_only(a)
        return
    if a.optimizer_only:
        optimizer_only(a)
        return
    if a.decode_only:
        decode_only(a)
        return
    import numpy as np
    import torch

    import dense_gpt_pretraining_nanochat_amd as nc
    from dense_gpt_pretraining_nanochat_amd import inputs
    from dense_gpt_pretraining_nanochat_amd.config import (PRESETS, SEEDS, TOKEN_LAW, flops_per_step,
                                                           flops_variants)

    c = PRESETS[a.workload]
    pseed, dseed = SEEDS[a.workload]
    cfg = nc.nc_config_from_depth(c.depth, c.vocab_size, c.seq_len, c.batch, c.dtype)
    nc.nc_set_lm_chunk_rows(a.lm_chunk_rows)
    step = nc.Step(cfg)
    step.init(pseed)
    tok, tgt = inputs.make_tokens(c.vocab_size, c.seq_len, c.batch, dseed, TOKEN_LAW[a.workload])
    tok_d, tgt_d = torch.from_numpy(tok).cuda(), torch.from_numpy(tgt).cuda()
    torch.cuda.synchronize()

    for _ in range(a.warmup):
        step.forward_backward(tok_d, tgt_d)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(s)
    for _ in range(a.steps):
        step.forward_backward(tok_d, tgt_d)
    ev1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sec = ev0.elapsed_time(ev1) / 1e3 / a.steps
    loss = float(step.loss.item())
    status = step.status()
    tokens = c.batch * c.seq_len
    fl = flops_per_step(c)
    out = {
        "metric": METRIC,
        "value": round(tokens / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic (seeded Zipf(1.1) token ids, random-init weights from nc_init_params)"
                if TOKEN_LAW[a.workload] == "zipf" else "synthetic (seeded uniform ids)",
        "config": {"workload": WORKLOAD_NAMES[a.workload], "batch": c.batch, "seq_len": c.seq_len,
                   "tokens_per_step": tokens, "parallelism": "none (one GPU)"},
        "mfu": round(fl / sec / (PEAK_BF16_TFLOPS * 1e12), 4),
        "flops_per_step": fl,
        "flops_variants": {k: float(v) for k, v in flops_variants(c).items()},
        "loss": loss,
        "device_status": status,
        "workspace_bytes": nc.nc_workspace_bytes(cfg, True),
        "lm_chunk_rows": nc.nc_lm_chunk_rows(cfg),
        "wall_s_timed": round(wall, 3),
    }
    in_step = roofline_after_steps(cfg, nc, torch, step, tok_d, tgt_d)
    if not a.no_eval:
        out["eval_bpb"] = bpb_timing(step, nc, torch, c, tok_d, tgt_d)
    if not a.no_optimizer:
        out["optimizer"] = optimizer_timing(step, nc, torch, c)
        step.opt_state = step.opt_ws = None
    if not a.no_decode:
        params = step.params
        step.ws = step.grads = None
        torch.cuda.empty_cache()
        out["decode"] = decode_timing(nc, torch, c, params, T0=min(1024, c.seq_len))
        del params
    del step
    torch.cuda.empty_cache()
    out["roofline"] = dominant_kernel_roofline(cfg, nc, torch)
    if in_step:
        out["roofline"]["after_step"] = in_step
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(a.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
