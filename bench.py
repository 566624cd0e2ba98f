"""Throughput of one tensor-parallel block shard on one MI355X.

A step is one forward pass of a 70B-shaped pre-norm block (h=8192, 64 query /
8 KV heads of 128, SwiGLU intermediate 28672, batch 4 x 2048 tokens, causal)
at t=8, with every rank's work run on this GPU one after another:

  RMSNorm(X) -> for each rank: QKV+RoPE GEMM, flash attention, o_proj GEMM
  -> shard-sum (+X) and RMSNorm(h1) in one pass -> for each rank: SwiGLU
  GEMM, down GEMM -> shard-sum (+h1).

The detail also times the sequence-parallel form of the same step (norms on
each rank's slice of every sequence, the sums as reduce-scatters onto those
slices), which computes the same result.

``value`` is the algorithmic bf16 flop rate of the step (2 flops per
multiply-add of every GEMM, causal attention counting only unmasked pairs)
over the wall time of the whole step, norms and sums included.  It equals the
per-shard rate, since the shards are identical work run back to back.

The JSON line also carries the dominant kernel's roofline (the SwiGLU
column-parallel GEMM, timed with HIP events around each of its launches on
the stream it runs on) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

REPO = Path(__file__).resolve().parent
sys.path.insert(0, str(REPO))

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16, published
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def block_flops(case, t: int) -> dict:
    """Algorithmic flops of one rank's share of the block, by kernel."""
    m, h, d = case.tokens, case.hidden, case.head_dim
    hq = case.heads // t
    group = case.heads // case.kv_heads
    hkv = (hq - 1) // group + 1 if hq >= group else 1
    f = case.inter // t
    pairs = case.seq * (case.seq + 1) / 2
    return {
        "qkv": 2.0 * m * h * (hq + 2 * hkv) * d,
        "attn_core": 4.0 * d * pairs * case.batch * hq,
        "o_proj": 2.0 * m * hq * d * h,
        "swiglu_gemm": 2.0 * m * h * 2 * f,
        "down_gemm": 2.0 * m * f * h,
    }


def block_backward_flops(case, t: int, saved: bool = False) -> float:
    """Algorithmic flops of one rank's share of the block's backward: the MLP's
    four backward GEMMs (12 m h f_t) and, unless the forward saved them, its
    recomputed gate/up GEMM (4 m h f_t); the attention's dO, core backward
    (2.5 times the core forward), dX, dW_qkv, dW_o and, unless saved, its
    recomputed forward (Q/K/V GEMM, core)."""
    f = block_flops(case, t)
    mlp = (12.0 if saved else 16.0) * case.tokens * case.hidden * (case.inter // t)
    attn = (2.0 if saved else 3.0) * f["qkv"] + 2.0 * f["o_proj"] + (2.5 if saved else 3.5) * f["attn_core"]
    return mlp + attn


TRAFFIC_FILE = REPO / "profiles" / "swiglu_gemm_traffic.json"
GEMM_SOURCE = REPO / "megatron_tensor_transformer_colwise_amd" / "csrc" / "gemm.hip"


def stored_traffic():
    """HBM bytes per launch of the SwiGLU GEMM from the committed counter runs,
    or None if the GEMM source changed since they were taken."""
    import json as _json

    from megatron_tensor_transformer_colwise_amd.pmc_traffic import source_hash

    if not TRAFFIC_FILE.exists():
        return None
    rec = _json.loads(TRAFFIC_FILE.read_text())
    if rec.get("source_sha256_16") != source_hash(str(GEMM_SOURCE)):
        return None
    return round(rec["traffic_bytes_per_launch"])


def cpu_baseline(case, w_host, budget_s: float = 20.0) -> dict:
    """The float64 oracle on a bounded sample of the workload: the same block
    (same weights, t ranks) over the first S tokens of one sequence, S doubled
    from 16 up to the sequence length, then over the first 2, 4, ... whole
    sequences, while the time stays within the budget."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from megatron_tensor_transformer_colwise_amd import inputs

    log("cpu baseline: widening weights to float64")
    W = {k: v.f64() for k, v in w_host.items() if k != "X"}
    x_all = w_host["X"]
    best = None
    s, nseq = 16, 1
    while True:
        sub = inputs.BlockCase(case.name + "-sample", nseq, s, case.hidden, case.heads, case.kv_heads,
                               case.head_dim, case.inter, case.t, case.rope_base, case.seed)
        Ws = dict(W)
        if nseq == 1:
            Ws["X"] = x_all.f32()[:s].astype(np.float64)
        else:  # the first nseq whole sequences
            Ws["X"] = x_all.f32()[:nseq * s].astype(np.float64)
        t0 = time.perf_counter()
        c0 = time.process_time()
        oracle.block(Ws["X"], Ws, sub)
        dt = time.perf_counter() - t0
        cpu = time.process_time() - c0
        fl = sum(block_flops(sub, case.t).values()) * case.t
        best = (s, nseq, dt, fl, cpu)
        log(f"cpu baseline: {nseq} x {s} tokens in {dt:.2f}s")
        if dt * 2.2 > budget_s or (s >= case.seq and nseq >= case.batch):
            break
        if s < case.seq:
            s *= 2
        else:
            nseq *= 2
    s, nseq, dt, fl, cpu = best
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "effective_cores": round(cpu / dt, 1),
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"{nseq} sequence(s) of {s} tokens through the same block (all {case.t} ranks, "
                  f"float64 numpy), {fl / 1e9:.1f} GFLOP in {dt:.2f} s",
    }


def _time(fn, reps=20, warm=5, before=None):
    """(median, min) milliseconds of fn over reps, each bracketed by events on
    the current stream; before() (e.g. a cache flush) runs outside the bracket."""
    import statistics

    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return statistics.median(ts), min(ts)


def _time_b2b(fn, reps=20, warm=5):
    """Mean milliseconds of fn over reps calls issued back to back between two
    events (no synchronisation between calls, as in a running model)."""
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / reps


def per_config_report(dev):
    """Per-call time and rate of every workload (one rank's call unless noted):
    median and minimum of 20 event-bracketed reps after 5 warm-ups.  Shard-sum
    reps are preceded by a 512 MiB write so the 256 MiB Infinity Cache holds
    none of their inputs."""
    import torch

    from megatron_tensor_transformer_colwise_amd import inputs, shard, tpshard as tp

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def flush():
        scratch.zero_()

    def emit(rec):
        print(json.dumps(rec), flush=True)

    def rate(fl, ms):
        return round(fl / ms / 1e9, 1)

    def sum_rec(fn, nbytes):
        med, mn = _time(fn, before=flush)
        return {"shard_sum_ms": round(med, 4), "shard_sum_min_ms": round(mn, 4),
                "shard_sum_gbs": round(nbytes / med / 1e6, 1),
                "shard_sum_pct_hbm": round(100.0 * nbytes / med / 1e6 / HBM_PEAK_GBS, 1)}

    # GPT-style GeLU MLP and Llama-8B SwiGLU MLP
    for name in ("gpt_gelu_mlp", "llama8b_swiglu_mlp"):
        case = inputs.CONFIGS[name]
        log(f"configs: {name}")
        dw = {k: v.torch().to(dev) for k, v in inputs.gen_mlp(case).items()}
        mlp = shard.MLPShards(dw["X"], dw, case.t, case.act)
        fl = 2.0 * case.tokens * case.hidden * case.f_shard * (3 if case.act == "swiglu" else 2)
        med, mn = _time(lambda: mlp.rank(0))
        b2b = _time_b2b(lambda: mlp.rank(0))
        rec = {"workload": name, "call": "tp_shard_mlp (one rank)", "ms": round(med, 4),
               "min_ms": round(mn, 4), "tflops": rate(fl, med),
               "pct_mfma_peak": round(100.0 * fl / med / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
               "b2b_ms": round(b2b, 4), "b2b_tflops": rate(fl, b2b),
               "b2b_pct_mfma_peak": round(100.0 * fl / b2b / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2)}
        gmed, gmn = _time(lambda: mlp.all_ranks_grouped())
        rec.update({"grouped_all_ranks_ms": round(gmed, 4), "grouped_min_ms": round(gmn, 4),
                    "grouped_tflops": rate(case.t * fl, gmed)})
        n = case.tokens * case.hidden
        rec.update(sum_rec(lambda: mlp.reduce(residual=None), (case.t + 1) * 4 * n))
        emit(rec)
        del mlp, dw

    # Llama-8B attention
    case = inputs.CONFIGS["llama8b_attn"]
    log("configs: llama8b_attn")
    dw = {k: v.torch().to(dev) for k, v in inputs.gen_attn(case).items()}
    at = shard.AttnShards(dw["X"], dw, case)
    fl = block_flops(inputs.BlockCase("a", case.batch, case.seq, case.hidden, case.heads, case.kv_heads,
                                      case.head_dim, case.hidden, case.t, case.rope_base, 0), case.t)
    afl = fl["qkv"] + fl["attn_core"] + fl["o_proj"]
    med, mn = _time(lambda: at.rank(0))
    b2b = _time_b2b(lambda: at.rank(0))
    rec = {"workload": "llama8b_attn", "call": "tp_shard_attn (one rank)", "ms": round(med, 4),
           "min_ms": round(mn, 4), "tflops": rate(afl, med),
           "pct_mfma_peak": round(100.0 * afl / med / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
           "b2b_ms": round(b2b, 4), "b2b_tflops": rate(afl, b2b),
           "b2b_pct_mfma_peak": round(100.0 * afl / b2b / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2)}
    n = case.tokens * case.hidden
    rec.update(sum_rec(lambda: at.reduce(residual=None), (case.t + 1) * 4 * n))
    emit(rec)
    del at, dw

    # 70B block at t = 8 and t = 16
    for name in ("llama70b_block_t8", "llama70b_block_t16"):
        case = inputs.CONFIGS[name]
        log(f"configs: {name}")
        dw = {k: v.torch().to(dev) for k, v in inputs.gen_block(case).items()}
        blk = shard.BlockShards(dw["X"], dw, case)
        fl = block_flops(case, case.t)
        afl = fl["qkv"] + fl["attn_core"] + fl["o_proj"]
        mfl = fl["swiglu_gemm"] + fl["down_gemm"]
        blk.norm_attn()
        blk.norm_mlp()
        ams, amn = _time(lambda: blk.attn.rank(0))
        mms, mmn = _time(lambda: blk.mlp.rank(0))
        ab2b = _time_b2b(lambda: blk.attn.rank(0))
        mb2b = _time_b2b(lambda: blk.mlp.rank(0))
        n = case.tokens * case.hidden
        srec = sum_rec(lambda: blk.mlp.reduce(residual=blk.attn.out, residual_dt="f32"),
                       (case.t + 2) * 4 * n)
        step, step_min = _time(lambda: blk.forward(), reps=5, warm=2)
        sp_step, sp_min = _time(lambda: blk.forward_sp(), reps=5, warm=2)
        rec = {"workload": name, "attn_call_ms": round(ams, 4), "attn_min_ms": round(amn, 4),
               "attn_tflops": rate(afl, ams),
               "attn_pct_mfma_peak": round(100.0 * afl / ams / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
               "mlp_call_ms": round(mms, 4), "mlp_min_ms": round(mmn, 4), "mlp_tflops": rate(mfl, mms),
               "mlp_pct_mfma_peak": round(100.0 * mfl / mms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
               "shard_aggregate_tflops": rate(afl + mfl, ams + mms),
               "attn_b2b_ms": round(ab2b, 4), "attn_b2b_tflops": rate(afl, ab2b),
               "mlp_b2b_ms": round(mb2b, 4), "mlp_b2b_tflops": rate(mfl, mb2b),
               "mlp_b2b_pct_mfma_peak": round(100.0 * mfl / mb2b / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2)}
        rec.update(srec)
        rec.update({"block_step_ms": round(step, 3), "block_step_min_ms": round(step_min, 3),
                    "block_step_tflops": rate(case.t * (afl + mfl), step),
                    "sequence_parallel_step_ms": round(sp_step, 3),
                    "sequence_parallel_step_tflops": rate(case.t * (afl + mfl), sp_step)})
        # the block's backward (after its forward), all ranks and both norm backwards
        dz = inputs.normal(93, 20, (case.tokens, case.hidden), 1.0, "bf16").torch().to(dev)
        blk.forward()
        blk.backward(dz)
        bstep, bmin = _time(lambda: blk.backward(dz), reps=3, warm=1)
        m, h = case.tokens, case.hidden
        nms, nmn = _time(lambda: tp.tp_shard_sum_rmsnorm_backward(
            case.t, m, h, list(blk.mlp.dx_partials), blk.attn.out, "f32", blk.g_mlp, case.eps, dz, "bf16", blk.dh1,
            blk.dh1_bf16, blk.dg_mlp, blk.norm_ws, blk.norm_ws_bytes))
        nbytes = (case.t * 4 + 4 + 2 + 4 + 2) * m * h
        bfl = case.t * block_backward_flops(case, case.t)
        rec.update({"block_backward_step_ms": round(bstep, 3), "block_backward_step_min_ms": round(bmin, 3),
                    "block_backward_step_tflops": rate(bfl, bstep),
                    "norm_backward_ms": round(nms, 4), "norm_backward_gbs": round(nbytes / nms / 1e6, 1)})
        # with the forward keeping its activations (no recomputation in the backward)
        fsv, _ = _time(lambda: blk.forward(save=True), reps=3, warm=1)
        blk.backward(dz)
        sstep, smin = _time(lambda: blk.backward(dz), reps=3, warm=1)
        sfl = case.t * block_backward_flops(case, case.t, saved=True)
        blk.forward()
        blk.backward_sp(dz)
        spb, _ = _time(lambda: blk.backward_sp(dz), reps=3, warm=1)
        rec.update({"sequence_parallel_backward_step_ms": round(spb, 3),
                    "sequence_parallel_backward_step_tflops": rate(bfl, spb)})
        rec.update({"saving_forward_step_ms": round(fsv, 3),
                    "saved_backward_step_ms": round(sstep, 3), "saved_backward_step_min_ms": round(smin, 3),
                    "saved_backward_step_tflops": rate(sfl, sstep)})
        emit(rec)
        del blk, dw, dz

    # packed single-stream block (the guide's [1, 1, 1, 3, 3] example, mlp
    # ratio 3): h = 3072, 24 heads of 128, 4608 tokens, no mask, t = 4
    h, heads, d, seq, t = 3072, 24, 128, 4608, 4
    log("configs: packed_single_stream")
    x = inputs.normal(81, 0, (seq, h), 1.0, "bf16").torch().to(dev)
    w_in = inputs.normal(81, 1, (9 * h, h), 0.02, "bf16").torch().to(dev)
    w_out = inputs.normal(81, 2, (h, 4 * h), 0.02, "bf16").torch().to(dev)
    ss = shard.SingleStreamShards(x, w_in, w_out, heads, d, 1, seq, t, 500000.0, causal=False)
    hr, mr, m = h // t, 3 * h // t, seq
    rfl = (2.0 * m * h * 3 * hr + 4.0 * d * seq * seq * (heads // t) + 2.0 * m * h * 2 * mr
           + 2.0 * m * (hr + mr) * h)
    rms, rmn = _time(lambda: ss.rank(0))
    fms, fmn = _time(lambda: ss.forward(), reps=10, warm=2)
    emit({"workload": "packed_single_stream", "call": "one rank: Q, K, V + RoPE and SwiGLU GEMMs from one packed "
          "buffer, attention, two out-projection partials", "ms": round(rms, 4), "min_ms": round(rmn, 4),
          "tflops": rate(rfl, rms), "pct_mfma_peak": round(100.0 * rfl / rms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
          "all_ranks_and_sum_ms": round(fms, 4), "all_ranks_tflops": rate(t * rfl, fms),
          "shape": f"h={h}, {heads} heads of {d}, mlp {3 * h}, {seq} tokens, t={t}, no mask"})
    del ss, x, w_in, w_out

    # vocabulary-parallel output layer + cross-entropy: h = 4096, vocabulary
    # 128256 over t = 4 ranks, 4096 tokens (the Llama-8B shapes of the other
    # workloads), labels seeded uniform
    h, v, m, t = 4096, 128256, 4096, 4
    log("configs: vocab_parallel_ce")
    x = inputs.normal(82, 0, (m, h), 1.0, "bf16").torch().to(dev)
    w = inputs.normal(82, 1, (v, h), 0.02, "bf16").torch().to(dev)
    import numpy as _np
    labels = torch.from_numpy(_np.random.default_rng(82).integers(0, v, m).astype(_np.int32)).to(dev)
    ce = shard.VocabParallelCE(x, w, t)
    n = v // t
    gfl = 2.0 * m * h * n
    rms, rmn = _time(lambda: ce.rank(0, labels))
    sms, smn = _time(lambda: tp.tp_ce_stats(m, n, 0, ce.logits, labels, ce.stats[0]))
    fms, fmn = _time(lambda: ce.forward(labels), reps=10, warm=2)
    emit({"workload": "vocab_parallel_ce", "call": "one rank: logits GEMM (float32) + max/sum/label statistics",
          "ms": round(rms, 4), "min_ms": round(rmn, 4), "tflops": rate(gfl, rms),
          "pct_mfma_peak": round(100.0 * gfl / rms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
          "stats_ms": round(sms, 4), "stats_gbs": round(4.0 * m * n / sms / 1e6, 1),
          "all_ranks_and_combine_ms": round(fms, 4), "all_ranks_tflops": rate(t * gfl, fms),
          "shape": f"h={h}, vocabulary {v} over t={t}, {m} tokens"})
    del ce, x, w

    # backward of one rank's SwiGLU MLP at the 70B block's shape (t = 8)
    case = inputs.MLPCase("llama70b_mlp_t8", 8192, 8192, 28672, 8, "swiglu", "bf16", seed=83)
    log("configs: llama70b_mlp_backward_t8")
    dw = {k: v.torch().to(dev) for k, v in inputs.gen_mlp(case).items()}
    dz = inputs.normal(83, 9, (case.tokens, case.hidden), 1.0, "bf16").torch().to(dev)
    mlp = shard.MLPShards(dw["X"], dw, case.t, "swiglu")
    m, h, f = case.tokens, case.hidden, case.f_shard
    bwd_fl = 2.0 * m * h * f * (1 + 2 + 1 + 2)      # dY, dX (2f), dW_out, dW_in (2f)
    rec_fl = 2.0 * m * h * 2 * f                    # the recomputed pre-activation
    bms, bmn = _time(lambda: mlp.backward_rank(0, dz), reps=10, warm=3)
    emit({"workload": "llama70b_mlp_backward_t8", "call": "tp_shard_mlp_backward (one rank, SwiGLU)",
          "ms": round(bms, 4), "min_ms": round(bmn, 4), "tflops": rate(bwd_fl + rec_fl, bms),
          "pct_mfma_peak": round(100.0 * (bwd_fl + rec_fl) / bms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
          "backward_only_tflops": rate(bwd_fl, bms),
          "shape": f"m={m}, h={h}, f_shard={f} (t=8), weight gradients float32"})
    del mlp, dw, dz

    # backward of one rank's attention at the 70B block's shape (t = 8: 8 query
    # heads, 1 KV head of 128, h = 8192, 4 sequences of 2048, causal); a
    # one-rank layer of that shape stands for the rank
    case, dw, dz, at = attn_backward_case(inputs, shard, dev)
    log("configs: llama70b_attn_backward_t8")
    fl = attn_backward_flops(case)
    bms, bmn = _time(lambda: at.backward_rank(0, dz), reps=10, warm=3)
    rk = at.ranks[0]
    core_in = attn_core_buffers(tp, at, case, dev, dz)
    cms, cmn = _time(lambda: core_in["run"](), reps=10, warm=3)
    emit({"workload": "llama70b_attn_backward_t8",
          "call": "tp_shard_attn_backward (one rank: forward recomputed, dO, core backward, dX, dW_qkv, dW_o)",
          "ms": round(bms, 4), "min_ms": round(bmn, 4), "tflops": rate(fl["total"], bms),
          "pct_mfma_peak": round(100.0 * fl["total"] / bms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
          "backward_only_tflops": rate(fl["backward"], bms),
          "core_call": "tp_flash_attn_backward (D, transposes, dQ, dK/dV, sum)", "core_ms": round(cms, 4),
          "core_min_ms": round(cmn, 4), "core_tflops": rate(fl["core_backward"], cms),
          "core_pct_mfma_peak": round(100.0 * fl["core_backward"] / cms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
          "shape": f"batch={case.batch}, seq={case.seq}, h={case.hidden}, hq={rk.hq}, hkv={rk.hkv}, d=128, "
                   "causal, weight gradients float32"})
    del at, dw, dz, core_in
    del scratch


def attn_backward_case(inputs, shard, dev):
    """One rank of the 70B attention at t = 8 (8 query heads, 1 KV head,
    h = 8192, 4 x 2048 tokens) with a seeded output gradient."""
    case = inputs.AttnCase("llama70b_attn_rank_t8", 4, 2048, 8192, 8, 1, 128, 1, 500000.0, seed=84)
    dw = {k: v.torch().to(dev) for k, v in inputs.gen_attn(case).items()}
    dz = inputs.normal(84, 9, (case.tokens, case.hidden), 1.0, "bf16").torch().to(dev)
    return case, dw, dz, shard.AttnShards(dw["X"], dw, case)


def attn_backward_flops(case) -> dict:
    """Algorithmic flops of one rank's attention backward: the recomputed
    forward (QKV GEMM, attention core), the dO GEMM, the core backward
    (dP, dV, dQ, dK over the causal pairs, plus the recomputed scores: 5
    products of 2 d flops per pair) and the dX, dW_qkv, dW_o GEMMs."""
    m, h, d = case.tokens, case.hidden, case.head_dim
    hq, hkv = case.heads // case.t, max(1, case.kv_heads // case.t)
    n = (hq + 2 * hkv) * d
    pairs = case.seq * (case.seq + 1) / 2 * case.batch * hq
    fwd = 2.0 * m * h * n + 4.0 * d * pairs
    core = 10.0 * d * pairs
    bwd = 2.0 * m * h * hq * d + core + 2.0 * m * n * h + 2.0 * m * h * n + 2.0 * m * h * hq * d
    return {"total": fwd + bwd, "backward": bwd, "core_backward": core}


def attn_core_buffers(tp, at, case, dev, dz):
    """The core backward alone on the rank's recomputed forward (run the
    sublayer backward once first so Q, K, V^T, O, LSE and dO are in its
    workspace)."""
    import torch

    rk = at.ranks[0]
    b, s, d = case.batch, case.seq, case.head_dim
    m = b * s
    n = (rk.hq + 2 * rk.hkv) * d
    sp = (s + 63) // 64 * 64
    core_bytes = tp.tp_flash_attn_backward_workspace_bytes(b, s, rk.hq, rk.hkv, d)
    q = torch.empty(m, rk.hq * d, dtype=torch.bfloat16, device=dev)
    k = torch.empty(m, rk.hkv * d, dtype=torch.bfloat16, device=dev)
    vt = torch.zeros(b, rk.hkv, d, sp, dtype=torch.bfloat16, device=dev)
    o = torch.empty(m, rk.hq * d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(b, rk.hq, sp, dtype=torch.float32, device=dev)
    do = torch.empty(m, rk.hq * d, dtype=torch.bfloat16, device=dev)
    tp.tp_qkv_rope(b, s, case.hidden, rk.hq, rk.hkv, d, case.rope_base, at.x, rk.w_qkv, q, k, vt)
    tp.tp_flash_attn_lse(b, s, rk.hq, rk.hkv, d, True, q, k, vt, o, lse)
    wo_t = torch.empty(rk.hq * d, case.hidden, dtype=torch.bfloat16, device=dev)
    tp.tp_transpose(case.hidden, rk.hq * d, rk.w_o, wo_t)
    tp.tp_colwise("none", "bf16", m, case.hidden, rk.hq * d, dz, wo_t, do)
    ws = torch.empty(core_bytes, dtype=torch.uint8, device=dev)
    dqkv = torch.empty(m, n, dtype=torch.bfloat16, device=dev)

    def run():
        tp.tp_flash_attn_backward(b, s, rk.hq, rk.hkv, d, case.rope_base, True, q, k, vt, o, lse, do, ws,
                                  core_bytes, dqkv, n)
    return {"run": run, "keep": (q, k, vt, o, lse, do, ws, dqkv, wo_t)}


def kernel_replay(blk, case, fl, stream, steps=3) -> dict:
    """Per-kernel average duration and roofline fraction in a replay of the
    step (after the timed region) in which every kernel launch is bracketed by
    HIP events on the stream it runs on; attention runs as its three component
    calls, the kernels tp_shard_attn launches.  GEMMs and attention are priced
    against the bf16 MFMA peak, the norms and sums (HBM-bound) against HBM."""
    import torch

    t = case.t
    n = case.tokens * case.hidden
    work = {  # name -> (amount per launch, unit, peak)
        "rmsnorm": (4 * n, "GB/s", HBM_PEAK_GBS),
        "qkv_rope": (fl["qkv"], "TFLOP/s", MFMA_BF16_PEAK_TFLOPS),
        "flash_attn": (fl["attn_core"], "TFLOP/s", MFMA_BF16_PEAK_TFLOPS),
        "o_proj": (fl["o_proj"], "TFLOP/s", MFMA_BF16_PEAK_TFLOPS),
        "sum_rmsnorm": ((4 * t + 8) * n, "GB/s", HBM_PEAK_GBS),
        "swiglu_gemm": (fl["swiglu_gemm"], "TFLOP/s", MFMA_BF16_PEAK_TFLOPS),
        "down_gemm": (fl["down_gemm"], "TFLOP/s", MFMA_BF16_PEAK_TFLOPS),
        "shard_sum": ((t + 2) * 4 * n, "GB/s", HBM_PEAK_GBS),
    }
    evs = {k: [] for k in work}
    open_ev = []

    def mark(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        if name is not None:
            open_ev.append((name, e))
        else:
            nm, e0 = open_ev.pop()
            evs[nm].append((e0, e))

    def timed(name, fn):
        mark(name)
        fn()
        mark(None)

    attn, mlp = blk.attn, blk.mlp
    for _ in range(steps):
        timed("rmsnorm", blk.norm_attn)
        for r in range(t):
            attn.rank_parts(r, mark=mark)
        timed("sum_rmsnorm", blk.sum_norm_mlp)
        for r in range(t):
            timed("swiglu_gemm", lambda: mlp.colwise(r))
            timed("down_gemm", lambda: mlp.rowwise(r))
        timed("shard_sum", lambda: mlp.reduce(residual=attn.out, residual_dt="f32"))
    torch.cuda.synchronize()
    out = {}
    for k, (amount, unit, peak) in work.items():
        us = 1e3 * sum(a.elapsed_time(b) for a, b in evs[k]) / len(evs[k])
        ach = amount / us / (1e6 if unit == "TFLOP/s" else 1e3)
        out[k] = {"avg_us": round(us, 2), "achieved": round(ach, 1), "peak": peak, "unit": unit,
                  "frac": round(ach / peak, 4), "launches": len(evs[k])}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama70b_block_t8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--configs", action="store_true",
                    help="per-call report for every workload (one JSON line each) instead of the step")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="launch a 256 MiB copy, then one step of the block (for counter runs)")
    ap.add_argument("--bwd-pass", action="store_true",
                    help="run one rank's SwiGLU MLP backward and attention backward at the 70B t=8 shape four "
                         "times each (for a kernel trace)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch

    from megatron_tensor_transformer_colwise_amd import inputs, shard, tpshard as tp

    if not tp.LIB_PATH.exists():
        import __graft_entry__

        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tp.tp_device_check()

    if args.configs:
        per_config_report(dev)
        return

    if args.bwd_pass:
        case = inputs.MLPCase("llama70b_mlp_t8", 8192, 8192, 28672, 8, "swiglu", "bf16", seed=83)
        dw = {k: v.torch().to(dev) for k, v in inputs.gen_mlp(case).items()}
        dz = inputs.normal(83, 9, (case.tokens, case.hidden), 1.0, "bf16").torch().to(dev)
        mlp = shard.MLPShards(dw["X"], dw, case.t, "swiglu")
        for _ in range(4):
            mlp.backward_rank(0, dz)
        torch.cuda.synchronize()
        log("MLP backward pass done")
        del mlp, dw, dz
        _, dw, dz, at = attn_backward_case(inputs, shard, dev)
        for _ in range(4):
            at.backward_rank(0, dz)
        torch.cuda.synchronize()
        log("attention backward pass done")
        return

    case = inputs.CONFIGS[args.config]
    t = case.t
    log(f"generating inputs for {case.name}")
    t0 = time.time()
    w = inputs.gen_block(case)
    log(f"inputs drawn in {time.time() - t0:.1f}s; uploading")
    dw = {k: v.torch().to(dev) for k, v in w.items()}
    blk = shard.BlockShards(dw["X"], dw, case)
    mlp, attn = blk.mlp, blk.attn
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log("weights sharded")

    if args.pmc_pass:
        # a plain copy of known size (shard-sum of one partial: 256 MiB read,
        # 256 MiB written), then the dominant kernel at the measured shape
        n = 64 << 20
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            tp.tp_shard_sum(1, n, [src], None, "f32", dst)
        torch.cuda.synchronize()
        blk.forward()  # one step: every kernel of the block, all ranks
        torch.cuda.synchronize()
        log("pmc pass done")
        return

    ev_pairs = []

    def step(record: bool):
        blk.norm_attn()
        for r in range(t):
            attn.rank(r)
        blk.sum_norm_mlp()
        for r in range(t):
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                mlp.colwise(r)
                e1.record(stream)
                ev_pairs.append((e0, e1))
            else:
                mlp.colwise(r)
            mlp.rowwise(r)
        mlp.reduce(residual=attn.out, residual_dt="f32")

    for i in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # timed region (the dominant kernel is bracketed by events inside it)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(True)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    fl = block_flops(case, t)
    step_flops = sum(fl.values()) * t
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    col_ms = sum(a.elapsed_time(b) for a, b in ev_pairs) / len(ev_pairs)
    col_tflops = fl["swiglu_gemm"] / (col_ms * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms, {value:.1f} TFLOP/s; swiglu gemm {col_ms * 1e3:.1f} us "
        f"= {col_tflops:.1f} TFLOP/s")

    # per-call breakdown (outside the timed region)
    def time_call(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    attn_ms = time_call(lambda: attn.rank(0))
    mlp_ms = time_call(lambda: mlp.rank(0))
    sum_ms = time_call(lambda: mlp.reduce(residual=attn.out, residual_dt="f32"))
    sum_norm_ms = time_call(lambda: blk.sum_norm_mlp())
    norm_ms = time_call(lambda: blk.norm_mlp())
    sp_ms = time_call(lambda: blk.forward_sp(), reps=3)
    n = case.tokens * case.hidden
    detail = {
        "attn_call_ms": round(attn_ms, 4),
        "attn_call_tflops": round((fl["qkv"] + fl["attn_core"] + fl["o_proj"]) / attn_ms / 1e9, 1),
        "mlp_call_ms": round(mlp_ms, 4),
        "mlp_call_tflops": round((fl["swiglu_gemm"] + fl["down_gemm"]) / mlp_ms / 1e9, 1),
        "shard_sum_ms": round(sum_ms, 4),
        "shard_sum_gbs": round((t + 2) * 4 * n / sum_ms / 1e6, 1),
        "sum_rmsnorm_ms": round(sum_norm_ms, 4),
        "sum_rmsnorm_gbs": round((4 * t + 8) * n / sum_norm_ms / 1e6, 1),
        "rmsnorm_f32_ms": round(norm_ms, 4),
        "rmsnorm_gbs": round(6 * n / norm_ms / 1e6, 1),
        "sequence_parallel_step_ms": round(sp_ms, 4),
        "sequence_parallel_tflops": round(step_flops / (sp_ms * 1e-3) / 1e12, 1),
    }
    log(f"detail {detail}")
    kernels = kernel_replay(blk, case, fl, stream, steps=3)
    log(f"kernels {kernels}")

    out = {
        "metric": "TFLOP/s per TP shard (MLP + attention, bf16) and % of MFMA bf16 peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs and weights, no checkpoint)",
        "pct_of_mfma_peak": round(100.0 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "config": {
            "workload": f"{case.name}: 70B-shaped block shard, h={case.hidden}, heads {case.heads}/"
                        f"{case.kv_heads}x{case.head_dim}, SwiGLU {case.inter}, t={t} (all ranks "
                        f"on one GPU), batch {case.batch} x seq {case.seq}, causal",
            "global_batch": case.batch,
            "seq_len": case.seq,
            "tp": t,
            "parallelism": f"tp{t} (ranks serialised on one GPU)",
        },
        "roofline": {
            "kernel": "gemm16_kernel<SWIGLU, 256> (column-parallel W1|W3 GEMM + SwiGLU, main and split-k launches)",
            "bound": "mfma",
            "achieved": round(col_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(col_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": stored_traffic(),
            "avg_launch_us": round(col_ms * 1e3, 2),
            "flops_per_launch": fl["swiglu_gemm"],
            "algorithmic_bytes_per_launch": 2 * (case.tokens * case.hidden
                                                 + 2 * (case.inter // t) * case.hidden
                                                 + case.tokens * (case.inter // t)),
        },
        "attention_roofline": {
            "kernel": "flash_attn_kernel (causal GQA flash attention forward, one rank's heads)",
            "bound": "mfma",
            **{k: kernels["flash_attn"][k] for k in ("achieved", "peak", "unit", "frac", "avg_us")},
        },
        "kernels": kernels,
        "detail": detail,
    }
    if not args.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0:
        out["cpu_baseline"] = cpu_baseline(case, w, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
