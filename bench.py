"""Training-step throughput of the gfx950 GPT path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2_124m]

One step = A x (forward_loss + backward) on micro-batches of B x T synthetic
token ids, then one AdamW update (global-norm clip, decoupled weight decay).
The default workload is GPT-2 124M (12 layers, 12 heads, n_embd 768, vocab
50257 padded to 50304), B 12, T 1024, A 5, bf16 GEMM/attention operands with
fp32 master weights: the configuration of the nanoGPT pages' GPT-2
reproduction with gradient accumulation. Inputs are generated on the host
and copied to the device before timing; the timed region holds only the
library's kernels. Prints one JSON line.

MFU uses the conventional count of 6N + 12 L d T FLOPs per token (N = parameters
without the position embedding) against 2.5 PFLOP/s dense bf16.

    python bench.py --decode [--prompt 128] [--new 256] [--temperature 0.8] [--top-k 40]

measures generation instead: a prefill of B prompts, then --new decode steps, each
one token per sequence through the key/value cache and one sampling launch, the
sampled tokens fed straight back on the device. Prints one JSON line with decode
tokens/s and the HBM roofline of a decode step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15        # dense bf16 MFMA, FLOP/s
PEAK_FP32 = 157.3e12      # dense fp32 MFMA
PEAK_HBM = 8.0e12         # bytes/s


def flops_per_token(cfg) -> float:
    """6N + 12 L d T with N the parameters that multiply activations: all but the
    position table (GPT-2: the tied wte counts once, as the lm_head); for the
    microGPT block, its matrices and its own lm_head (the wte gather is no product)."""
    d, L, T, V = cfg.n_embd, cfg.n_layer, cfg.block_size, cfg.padded_vocab
    if getattr(cfg, "variant", "gpt2") == "microgpt":
        N = V * d + L * 12 * d * d
    else:
        n_params = V * d + T * d + L * (12 * d * d + 13 * d) + 2 * d
        N = n_params - T * d
    if getattr(cfg, "lora_rank", 0) > 0:
        # LoRA fine-tuning: forward 2N + 4 L d T, input gradients 2N + 8 L d T, and of
        # the weight gradients only the q and v blocks, 4 L d^2 (the adapters' own
        # products run once per step, not per token)
        return 4.0 * N + 12.0 * L * d * T + 4.0 * L * d * d
    return 6.0 * N + 12.0 * L * d * T


def blas_info():
    """(library, threads) of the BLAS NumPy calls, as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version') or ''}".strip(), int(i.get("num_threads", 1))
    except Exception:
        pass
    return "unknown", 0


def cpu_baseline(cfg, params, batches, n_seq: int, dropout: float = 0.0):
    """The oracle as it stands, in float32, on the first micro-batch of the workload
    (its first n_seq sequences: the whole micro-batch by default) and one AdamW
    update of every parameter. The step rate is extrapolated to the workload's A
    micro-batches per update: tokens of A micro-batches over A times the measured
    forward + backward plus the measured clip + AdamW."""
    from oracle import gpt_oracle as O
    tok, tgt = batches[0]
    tok, tgt = tok[:n_seq], tgt[:n_seq]
    A = len(batches)
    lib, threads = blas_info()
    tr = O.Trainer(params, cfg, dtype=np.float32, dropout=O.Dropout(dropout, 1337) if dropout > 0 else None)
    marks = []
    t0 = time.perf_counter()
    tr.step([(tok, tgt)], progress=lambda i, l: marks.append(time.perf_counter()))
    t2 = time.perf_counter()
    t_mb, t_opt = marks[0] - t0, t2 - marks[0]
    step_s = A * t_mb + t_opt
    return {"value": round(A * tok.size / step_s, 3), "unit": "tokens/s", "cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"float32 oracle: 1 micro-batch of {tok.shape[0]} x {tok.shape[1]} tokens forward + backward "
                      f"({t_mb:.1f} s) and one clip + AdamW over all {O.n_params(cfg)} parameters ({t_opt:.1f} s); "
                      f"rate for a step of {A} micro-batches = {A} x {t_mb:.1f} + {t_opt:.1f} s",
            "blas": lib, "blas_threads": threads,
            "note": "per-sequence loops in NumPy: only the BLAS matrix products use several threads"}


def decode_bytes(cfg, B: int, length: int, op_bytes: int) -> float:
    """Algorithmic HBM bytes of one decode step at cache length `length` (the new
    position included): every weight read once in operand type (the tied wte for the
    lm_head, 12 d^2 per layer), biases and LayerNorm parameters in fp32, the keys and
    values of `length` positions read and one position written per layer and
    sequence, the embedding rows, the fp32 logits written."""
    d, L, V = cfg.n_embd, cfg.n_layer, cfg.padded_vocab
    weights = (V * d + L * 12 * d * d) * op_bytes + (L * 13 * d + 2 * d) * 4
    kv = L * B * (length + 1) * 2 * d * op_bytes
    rows = B * 2 * d * 4 + B * V * 4
    return float(weights + kv + rows)


def bench_decode(a, cfg) -> int:
    import torch
    from transformer_lm_gpt_amd import workloads as W
    from transformer_lm_gpt_amd.binding import GPT
    B, T0, n = cfg.batch, a.prompt, a.new
    if T0 < 1 or T0 + n > cfg.block_size:
        print(f"--prompt {T0} + --new {n} exceeds block_size {cfg.block_size}", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng)
    prompt, _ = W.make_batch(cfg, drng, B=B, T=T0)
    urng = np.random.default_rng(7)
    uni = torch.from_numpy(urng.random((n, B)).astype(np.float32)).cuda()
    tok = torch.from_numpy(prompt).cuda()
    gpu = GPT(cfg, a.precision, device="cuda:0", kv_cache=True)
    gpu.load_params(params)
    stream = torch.cuda.current_stream()

    def generate():
        z = gpu.prefill(tok)
        t = gpu.sample(z, a.temperature, a.top_k, None if a.temperature <= 0 else uni[0], out=gpu.decode_tokens())
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(1, n + 1):
            z = gpu.decode(t)
            t = gpu.sample(z, a.temperature, a.top_k, None if a.temperature <= 0 else uni[s % n], out=t)
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record(stream)
        return e0, e1, t

    generate()                                        # warm-up
    gpu.sync()
    torch.cuda.synchronize()
    ep = torch.cuda.Event(enable_timing=True)
    ep.record(stream)
    e0, e1, t = generate()
    torch.cuda.synchronize()
    gpu.sync()
    dec_ms = e0.elapsed_time(e1)
    pre_ms = ep.elapsed_time(e0)
    step_ms = dec_ms / n
    op = 2 if a.precision == "bf16" else 4
    bytes_avg = sum(decode_bytes(cfg, B, T0 + s, op) for s in range(n)) / n
    achieved = bytes_avg / (step_ms / 1e3)
    cpu = None
    if a.cpu_seqs > 0:
        from oracle import gpt_oracle as O
        t0 = time.perf_counter()
        O.generate(params, prompt[:1], cfg, 2, a.temperature, a.top_k, np.full((2, 1), 0.5))
        dt = time.perf_counter() - t0
        cpu = {"value": round(2 / dt, 3), "unit": "tokens/s", "cores": os.cpu_count(), "kind": "oracle",
               "sample": f"1 sequence, prompt {T0}, 2 new tokens by full float64 recomputation ({dt:.1f} s)"}
    out = {
        "metric": f"decode tokens/sec with a key/value cache, {cfg.name}, 1 MI355X",
        "value": round(B * n / (dec_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": 1,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": a.precision,
        "data": f"synthetic prompts (seeded, {cfg.data}), random-init weights N(0,{cfg.init_std})",
        "config": {"workload": f"{cfg.name}: L{cfg.n_layer} H{cfg.n_head} d{cfg.n_embd} V{cfg.padded_vocab} "
                               f"B{B} prompt {T0} + {n} new, temperature {a.temperature}, top-k {a.top_k}"},
        "prefill_ms": round(pre_ms, 3),
        "roofline": {"kernel": "one decode step (all layers, lm_head, sampling)", "bound": "hbm",
                     "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM, 4), "traffic": None,
                     "bytes_per_step": round(bytes_avg)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    gpu.close()
    return 0


def traffic_of(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (profiles/traffic.json), or None when the counters were taken on another workload
    or its source has changed since (the summary records a hash of the source file)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("workload") != workload:
        return None
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return rec["bytes_per_launch"]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2_124m")
    ap.add_argument("--precision", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--kernel", default="gemm_wgrad",
                    help="kernel family whose launches are timed for the roofline line "
                         "(gemm_wgrad: the grouped weight-gradient GEMM, the step's largest kernel; lm_head_fwd)")
    ap.add_argument("--cpu-seqs", type=int, default=12,
                    help="sequences of the first micro-batch in the oracle's timed sample (0: skip)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout rate of the timed model (the GPT-2 124M workload uses 0)")
    ap.add_argument("--decode", action="store_true", help="measure generation with the key/value cache")
    ap.add_argument("--prompt", type=int, default=128, help="--decode: prompt length")
    ap.add_argument("--new", type=int, default=256, help="--decode: generated tokens per sequence")
    ap.add_argument("--temperature", type=float, default=0.8, help="--decode: sampling temperature")
    ap.add_argument("--top-k", type=int, default=40, help="--decode: top-k cut (0: none)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run 3 plain device copies of this many bytes (calibrates the HBM byte counters)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the data-parallel all-reduce "
              f"is not part of this build", file=sys.stderr)
        return 2

    import torch
    from transformer_lm_gpt_amd import workloads as W
    from transformer_lm_gpt_amd.binding import GPT

    if a.copy_bytes > 0:
        src = torch.ones(a.copy_bytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.copy_bytes, "copies": 3}), flush=True)
        return 0

    cfg = W.CONFIGS[a.workload]
    if a.decode:
        return bench_decode(a, cfg)
    B, T, A = cfg.batch, cfg.block_size, cfg.grad_accum
    torch.cuda.set_device(0)
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng)
    n_steps = a.warmup + a.steps
    host_batches = [W.make_step_batches(cfg, drng) for _ in range(min(n_steps, 4))]
    dev_batches = [[(torch.from_numpy(t).cuda(), torch.from_numpy(y).cuda()) for t, y in s] for s in host_batches]

    gpu = GPT(cfg, a.precision, device="cuda:0", dropout=a.dropout)
    gpu.load_params(params)
    if a.dropout > 0:
        gpu.set_dropout_seed(1337, 0)
    loss = torch.zeros(A, dtype=torch.float32, device="cuda:0")
    norm = torch.zeros(1, dtype=torch.float32, device="cuda:0")

    def step(i):
        for j, (t, y) in enumerate(dev_batches[i % len(dev_batches)]):
            gpu.forward_loss(t, y, loss_out=loss[j:j + 1])
            gpu.backward()
        gpu.adamw_step(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.grad_clip, norm_out=norm)

    for i in range(a.warmup):
        step(i)
    gpu.sync()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    gpu.timer_enable(a.kernel)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(a.steps):
        step(a.warmup + i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms, kern_n = gpu.timer_read()
    gpu.timer_disable()
    gpu.sync()
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps)]
    total_ms = ev[0].elapsed_time(ev[-1])
    final_loss = float(loss.mean().item())
    if not math.isfinite(final_loss):
        raise RuntimeError(f"non-finite loss {final_loss}")

    tokens_per_step = B * T * A
    ms = total_ms / a.steps
    tps = tokens_per_step / (ms / 1e3)
    ftok = flops_per_token(cfg)
    peak = PEAK_BF16 if a.precision == "bf16" else PEAK_FP32
    mfu = tps * ftok / peak
    causal_ftok = ftok - 6.0 * cfg.n_layer * cfg.n_embd * T

    # roofline of the timed kernel family
    roof = None
    if kern_n:
        avg_ms = kern_ms / kern_n
        d, L, Vp = cfg.n_embd, cfg.n_layer, cfg.padded_vocab
        if a.kernel == "lm_head_fwd":
            work = 2.0 * B * T * Vp * d                                  # FLOPs per launch
            roof = {"kernel": "lm_head forward GEMM (gemm_dma_kernel 192x192, bf16, store epilogue)", "bound": "mfma",
                    "achieved": round(work / (avg_ms / 1e3) / 1e12, 2), "peak": peak / 1e12, "unit": "TFLOP/s",
                    "frac": round(work / (avg_ms / 1e3) / peak, 4), "traffic": None,
                    "avg_launch_ms": round(avg_ms, 4), "launches": kern_n,
                    "work_per_launch": f"2*M*Vp*d = {work:.4g} FLOP, M = {B * T}"}
        elif a.kernel == "gemm_wgrad" and a.precision == "bf16":
            # every weight gradient of a micro-batch, K = B*T tokens each: one grouped
            # launch per micro-batch where every tensor's shape allows it, else one per tensor
            mbs = a.steps * A
            lora = cfg.lora_rank > 0                                     # q and v blocks only
            work = 2.0 * B * T * (2 * L * d * d if lora else Vp * d + L * 12 * d * d)   # FLOPs per micro-batch
            per_mb = kern_ms / mbs
            grouped = kern_n == mbs
            roof = {"kernel": ("grouped weight-gradient GEMM (gemm_group_wide_kernel: 256x256 tiles on 4 wavefronts of "
                               "128x128, + group_fixup_kernel; bf16 operands, fp32 accumulate)") if grouped else
                              f"weight-gradient GEMMs, {kern_n / mbs:g} launches per micro-batch",
                    "bound": "mfma",
                    "achieved": round(work / (per_mb / 1e3) / 1e12, 2), "peak": peak / 1e12, "unit": "TFLOP/s",
                    "frac": round(work / (per_mb / 1e3) / peak, 4),
                    "traffic": traffic_of("gemm_group_wide_kernel", cfg.name) if grouped else None,
                    "avg_launch_ms": round(avg_ms, 4), "launches": kern_n,
                    ("work_per_launch" if grouped else "work_per_micro_batch"):
                        (f"2*M*(2*L*d^2) = {work:.4g} FLOP" if lora else f"2*M*(Vp*d + 12*L*d^2) = {work:.4g} FLOP")
                        + f", M = {B * T}"}
        else:
            roof = {"kernel": a.kernel, "avg_launch_ms": round(avg_ms, 4), "launches": kern_n}

    cpu = None
    if a.cpu_seqs > 0:
        cpu = cpu_baseline(cfg, params, host_batches[0], a.cpu_seqs, a.dropout)

    metric = ("training tokens/sec and MFU, GPT-2 124M fwd+bwd+AdamW, T=1024, 1 MI355X"
              if cfg.name == "gpt2_124m" and a.dropout == 0
              else f"training tokens/sec and MFU, {cfg.name} fwd+bwd+AdamW, T={T}, 1 MI355X"
                   + (f", dropout {a.dropout}" if a.dropout else ""))
    ids = {"zipf_batch": f"Zipf({cfg.zipf_s}) ids over {cfg.vocab_size}",
           "zipf_stream": f"windows of a Zipf({cfg.zipf_s}) id stream over {cfg.vocab_size}",
           "markov_stream": f"windows of an order-1 Markov id stream over {cfg.vocab_size}",
           "uniform": f"uniform ids over {cfg.vocab_size}"}[cfg.data]
    out = {
        "metric": metric,
        "value": round(tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": a.precision,
        "data": f"synthetic (seeded {ids}, random-init weights N(0,{cfg.init_std}))",
        "config": {"workload": f"{cfg.name}: L{cfg.n_layer} H{cfg.n_head} d{cfg.n_embd} V{cfg.vocab_size}"
                               f"(pad {cfg.padded_vocab}) B{B} T{T} accum{A}",
                   "global_batch": B * A, "seq_len": T, "tokens_per_step": tokens_per_step,
                   "dropout": a.dropout,
                   **({"lora_rank": cfg.lora_rank, "lora_alpha": cfg.lora_alpha, "lora_on": "q, v"}
                      if cfg.lora_rank else {})},
        "mfu": round(mfu, 4),
        "mfu_causal_exact": round(tps * causal_ftok / peak, 4),
        "achieved_tflops": round(tps * ftok / 1e12, 1),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 3) for q in (10, 50, 90)],
        "wall_s": round(wall, 3),
        "final_loss": round(final_loss, 5),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    gpu.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
