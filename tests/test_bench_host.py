"""Host-side pieces of bench.py (no GPU): the FLOP count behind MFU and the guard on the
recorded HBM traffic."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from transformer_lm_gpt_amd import workloads as W  # noqa: E402


def test_flops_per_token_gpt2_124m():
    # 6N + 12 L d T with N = parameters without wpe: 123,689,472 at Vp 50304, d 768, L 12
    cfg = W.CONFIGS["gpt2_124m"]
    d, L, T = cfg.n_embd, cfg.n_layer, cfg.block_size
    assert bench.flops_per_token(cfg) == 6.0 * 123_689_472 + 12.0 * L * d * T
    assert abs(bench.flops_per_token(cfg) / 1e6 - 855.4) < 0.05


def test_traffic_only_for_its_workload_and_source():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)["gemm_group_wide_kernel"]
    got = bench.traffic_of("gemm_group_wide_kernel", rec["workload"])
    assert got in (None, rec["bytes_per_launch"])       # None once the source changed
    assert bench.traffic_of("gemm_group_wide_kernel", "char_6l") is None
    assert bench.traffic_of("no_such_kernel", rec["workload"]) is None


def test_flops_per_token_gpt2_124m_lora():
    # LoRA on q and v: 4N + 12 L d T + 4 L d^2 (no weight gradients but the q and v blocks)
    cfg = W.CONFIGS["gpt2_124m_lora"]
    d, L, T = cfg.n_embd, cfg.n_layer, cfg.block_size
    assert bench.flops_per_token(cfg) == 4.0 * 123_689_472 + 12.0 * L * d * T + 4.0 * L * d * d
    assert abs(bench.flops_per_token(cfg) / 1e6 - 636.3) < 0.05


def test_cpu_baseline_reports_cores_blas_and_a_whole_step():
    """The oracle's timed sample: float32, a micro-batch plus one AdamW update, the
    rate extrapolated to the workload's A micro-batches; os.cpu_count(), the BLAS
    library and its thread count reported apart (a toy size keeps this quick)."""
    import numpy as np
    cfg = W.CONFIGS["char_small"].with_(grad_accum=3)
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng)
    batches = W.make_step_batches(cfg, drng)
    out = bench.cpu_baseline(cfg, params, batches, n_seq=cfg.batch)
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s" and out["value"] > 0
    assert out["cores"] == os.cpu_count()
    assert isinstance(out["blas"], str) and out["blas_threads"] >= 0
    assert "float32" in out["sample"] and "3 micro-batches" in out["sample"]
