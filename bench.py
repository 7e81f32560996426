#!/usr/bin/env python3
"""Decode / prefill benchmark of the gfx950 Llama-2 decoder forward.

One step = one whole generate pass over the workload's batch: prompt tokens
already in HBM -> prefill -> sample -> decode steps, each followed by a sample
(and, for ragged prompts, the prompt forcing of the reference's generate
loop).  The host never synchronises inside a step.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from llama_decoder_forward_amd import configs, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published


def decode_bytes_per_step(w, B, L_avg):
    """Algorithmic HBM bytes of one decode step: every layer matrix and the
    output head once, the attended KV prefix once per KV head, the KV write."""
    hd = w.head_dim
    kv_read = B * L_avg * 2 * w.n_kv_heads * hd * 2 * w.n_layers
    kv_write = B * 2 * w.n_kv_heads * hd * 2 * w.n_layers
    return w.weight_bytes() + kv_read + kv_write


def product_bytes(w, B):
    """Algorithmic HBM bytes of one launch of each decode weight product at
    batch B (fp16): the weight matrix once, the B activation rows in (plus
    the RMSNorm weight where the norm runs inside the product), the outputs
    out (the residual read and written back for wo and w2, q and the K/V
    cache entries for wq|wk|wv, fp32 logits for the head)."""
    D, hd, F, V = w.dim, w.head_dim, w.ffn_hidden(), w.vocab_size
    qd, kvd = w.n_heads * hd, w.n_kv_heads * hd
    return {
        "qkv": 2 * ((qd + 2 * kvd) * D + B * D + D + B * (qd + 2 * kvd)),
        "o": 2 * (D * qd + B * qd + 2 * B * D),
        "w13": 2 * (2 * F * D + B * D + D + B * F),
        "w2": 2 * (D * F + B * F + 2 * B * D),
        "head": 2 * (V * D + B * D + D) + 4 * B * V,
    }


def prefill_product_flops(w, M):
    """Flops of the layer weight products of a prefill of M rows, by kind
    (all layers; the head runs on the last position only and is left out)."""
    D, hd, F = w.dim, w.head_dim, w.ffn_hidden()
    qd, kvd = w.n_heads * hd, w.n_kv_heads * hd
    per = {"qkv": (qd + 2 * kvd) * D, "o": D * qd, "w13": 2 * F * D, "w2": D * F}
    return {k: 2 * v * M * w.n_layers for k, v in per.items()}


def prefill_flops(w, B, T):
    """2 * params * tokens for the layer matrices, causal attention
    2 * B * H * d * T (T + 1) per layer, head at the last position."""
    lin = 2 * w.layer_params() * B * T * w.n_layers
    att = 2 * B * w.n_heads * w.head_dim * T * (T + 1) * w.n_layers
    head = 2 * w.vocab_size * w.dim * B
    return lin + att + head


def cpu_baseline(w, prompt, budget_s=15.0, max_steps=64):
    """The oracle (untuned) on this host, end to end on the whole model of
    the workload: one row, the prompt's prefill, then greedy decode steps
    until about budget_s seconds of decoding have run (at least two).  The
    value is the decode rate of that row (tok/s); rows of a batch would run
    one after another."""
    import oracle
    T0 = len(prompt)
    kw = w.model_kwargs(max_batch_size=1, max_seq_len=min(w.max_seq_len, T0 + max_steps + 1))
    t0 = time.perf_counter()
    m = oracle.Model(oracle.Cfg(**kw), w.weight_seed)
    t_create = time.perf_counter() - t0
    t0 = time.perf_counter()
    lg = m.forward(np.asarray(prompt, np.int32)[None], 0)
    t_prefill = time.perf_counter() - t0
    t0 = time.perf_counter()
    n = 0
    while n < max_steps and (n < 2 or time.perf_counter() - t0 < budget_s):
        lg = m.forward(np.asarray([[int(lg[0].argmax())]], np.int32), T0 + n)
        n += 1
    t_dec = time.perf_counter() - t0
    m.close()
    return {"value": n / t_dec, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole {w.n_layers}-layer model end to end on one row: {T0}-token prefill "
                      f"({t_prefill:.2f} s) then {n} greedy decode steps ({t_dec:.2f} s); value = decode "
                      f"tok/s of those steps; weights generated in {t_create:.1f} s (not timed)",
            "nproc": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "seconds_per_token_row": t_dec / n, "prefill_s": t_prefill}


def counter_traffic(w):
    """HBM bytes (fetched + written) per decode product launch from the
    committed counter summary of this workload, or None when there is none or
    the product kernels' sources changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"decode_products_traffic_{w.name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        k, sep, v = line.partition(":")
        if sep and v.split():
            vals[k.strip()] = v.split()[0]
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h"):
        with open(os.path.join(ROOT, "llama_decoder_forward_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("source_sha256_16") != h.hexdigest()[:16] or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=configs.L7B_BS1.name,
                    choices=sorted(k for k, v in configs.WORKLOADS.items() if v.dtype == configs.F16))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--second", default=configs.L70B_BS32.name,
                    help="a second workload measured in the same run (its decode and prefill rates go "
                         "into detail.second_workload); 'none' to skip")
    ap.add_argument("--profile-reps", type=int, default=5)
    ap.add_argument("--kv-block", type=int, default=0,
                    help="run with a paged KV cache of blocks of this many positions (a pool with room "
                         "for every row at max_seq_len) instead of the static cache")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device to device three times (a known-size kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the decoder's rows are independent, so more GPUs would run data-parallel replicas "
              "with no exchange, and that path is not built here.", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = configs.WORKLOADS[args.workload]
    out = measure(w, args.steps, args.warmup, args.profile_reps, args.kv_block)
    if args.second and args.second != "none" and args.second != w.name:
        # the metric's second configuration, measured in the same run: one
        # warm-up and one timed generate pass
        w2 = configs.WORKLOADS[args.second]
        o2 = measure(w2, 1, 1, 2, args.kv_block)
        d2 = o2["detail"]
        out["detail"]["second_workload"] = {
            "workload": w2.name, "batch": w2.batch, "generate_tok_s": o2["value"],
            "ms_per_generate_pass": o2["ms_per_step"],
            "decode_tok_s_incl_sampling": d2["decode_tok_s_incl_sampling"],
            "decode_roofline_tok_s": d2["decode_roofline_tok_s"],
            "decode_frac_of_roofline": d2["decode_frac_of_roofline"],
            "prefill_ms": d2["prefill_ms"], "prefill_tok_s": d2["prefill_tok_s"],
            "prefill_tflops": d2["prefill_tflops"],
            "prefill_frac_of_mfma": round(d2["prefill_tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
            "prefill_products_tflops": d2["prefill_products_tflops"],
            "decode_products": {k: o2["roofline"][k] for k in ("achieved", "frac", "avg_launch_us")},
            "profile_ms_per_decode_step": d2["profile_ms_per_decode_step"],
            "create_s": d2["create_s"],
        }
    if not args.no_cpu_baseline:
        T0 = out["detail"]["prefill_rows_per_batch_row"]
        prompt = synth.tokens(w.token_seed, 1, T0, w.vocab_size)[0]
        out["cpu_baseline"] = cpu_baseline(w, prompt[:16].tolist())
        if T0 > 16:
            out["cpu_baseline"]["sample"] += f" (the first 16 of the {T0} prompt tokens)"
    out["detail"].pop("prefill_rows_per_batch_row")
    print(json.dumps(out), flush=True)


def measure(w, n_steps, warmup, profile_reps, kv_block):
    """Time n_steps whole generate passes of workload w (after warmup ones)
    and profile its kernels; returns the bench line without cpu_baseline."""
    import torch
    from llama_decoder_forward_amd import binding as Bd

    B = w.batch
    ragged = bool(w.prompt_range)
    if ragged:
        lens = synth.prompt_lengths(w.token_seed, B, *w.prompt_range)
        T0 = int(lens.min())
        Tmax = int(lens.max())
    else:
        lens = np.full(B, w.prompt_len, np.int32)
        T0 = Tmax = w.prompt_len
    steps = w.decode_steps
    prompts = synth.tokens(w.token_seed, B, Tmax, w.vocab_size)
    uni = synth.uniforms(w.uniform_seed, steps + 1, B)
    temp, top_p = w.temperature, w.top_p

    t_create = time.perf_counter()
    if kv_block:
        nblk = B * -(-w.max_seq_len // kv_block)
        h = Bd.llm_create_paged(Bd.params_for(w), Bd.make_paging(kv_block, nblk), w.weight_seed)
    else:
        h = Bd.llm_create(Bd.params_for(w), w.weight_seed)
    t_create = time.perf_counter() - t_create
    stream = torch.cuda.ExternalStream(h.stream())

    # inputs resident in HBM before timing
    tok_dev = torch.from_numpy(np.ascontiguousarray(prompts[:, :T0])).cuda()
    uni_dev = torch.from_numpy(np.ascontiguousarray(uni)).cuda()
    S = w.max_seq_len
    force_tok = np.zeros((S, B), np.int32)
    force_mask = np.zeros((S, B), np.uint8)
    for b in range(B):
        force_tok[:lens[b], b] = prompts[b, :lens[b]]
        force_mask[T0:lens[b], b] = 1
    force_tok_dev = torch.from_numpy(force_tok).cuda()
    force_mask_dev = torch.from_numpy(force_mask).cuda()
    torch.cuda.synchronize()

    def generate(ev=None):
        h.prefill_d(tok_dev.data_ptr(), B, T0)
        h.sample_d(temp, top_p, uni_dev.data_ptr() if temp > 0 else 0, 0)
        if ev is not None:
            ev.record(stream)
        for i in range(steps):
            p = T0 + i
            if ragged and force_mask[p].any():
                h.set_tokens_d(p, force_tok_dev[p].data_ptr(), force_mask_dev[p].data_ptr())
            h.decode(p)
            h.sample_d(temp, top_p, uni_dev[i + 1].data_ptr() if temp > 0 else 0, 0)

    for _ in range(warmup):
        generate()
    h.sync()
    torch.cuda.synchronize()

    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    ev_pf = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps)]
    ev_st = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_start.record(stream)
    for k in range(n_steps):
        ev_st[k].record(stream)
        generate(ev_pf[k])
    ev_end.record(stream)
    h.sync()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev_start.elapsed_time(ev_end)
    prefill_ms = float(np.mean([ev_st[k].elapsed_time(ev_pf[k]) for k in range(n_steps)]))

    ms_per_step = wall * 1e3 / n_steps
    value = B * steps / (ms_per_step / 1e3)
    decode_ms = ms_per_step - prefill_ms
    decode_tok_s = B * steps / (decode_ms / 1e3)

    # live per-kernel-class timing of one decode step (HIP events on the
    # library's stream), at the last position of the generate pass
    prof = h.profile_decode(T0 + steps - 1, profile_reps)
    # the dominant kernel, the skinny GEMV of the decode weight products:
    # the products of a decode step in forward order, replayed from a
    # captured graph between two HIP events on the library's stream (and
    # each kind on its own for the breakdown)
    prod_us = h.profile_projections(profile_reps)
    # prefill kernels by class (eager, HIP events around every kernel); the
    # weight products' share of the prefill flops against the MFMA peak
    pf_prof = h.profile_prefill_d(tok_dev.data_ptr(), B, T0, 1)
    pf_gemm = prefill_product_flops(w, B * T0)
    pf_gemm_ms = sum(pf_prof[k] for k in pf_gemm)
    pf_gemm_tflops = sum(pf_gemm.values()) / (pf_gemm_ms / 1e3) / 1e12
    pbytes = product_bytes(w, B)
    per_step = {k: (1 if k == "head" else w.n_layers) for k in pbytes}
    launches = sum(per_step.values())
    step_prod_bytes = sum(per_step[k] * pbytes[k] for k in pbytes)
    step_prod_us = prod_us["step_order"] * launches
    achieved = step_prod_bytes / (step_prod_us / 1e6) / 1e9
    L_avg = T0 + steps / 2
    step_bytes = decode_bytes_per_step(w, B, L_avg)
    step_roof_tok_s = B * HBM_PEAK_GBS * 1e9 / step_bytes

    pf_flops = prefill_flops(w, B, T0)
    prefill_tok_s = B * T0 / (prefill_ms / 1e3)

    out = {
        "metric": "decode tok/s",
        "value": round(value, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if w.dtype == configs.F16 else "f32",
        "data": "synthetic: seeded SplitMix64 weights ~N(0,0.02), uniform prompt tokens",
        "config": {"workload": w.name, "batch": B, "prompt": T0 if not ragged else f"ragged {w.prompt_range}, prefill {T0}",
                   "decode_steps": steps, "temperature": temp, "top_p": top_p,
                   "layers": w.n_layers, "dim": w.dim, "heads": f"{w.n_heads}/{w.n_kv_heads}",
                   "ffn": w.ffn_hidden(), "vocab": w.vocab_size, "max_seq_len": S,
                   "kv_cache": f"paged, blocks of {kv_block}" if kv_block else "static"},
        "roofline": {"bound": "hbm",
                     "kernel": "gemm_skinny_kernel (decode weight products: wq|wk|wv, wo, w1|w3, w2, head)",
                     "scope": "the weight products of a decode step only, replayed from a captured graph; "
                              "the whole step (attention, sampling, launch gaps included) against the "
                              "step's roofline is detail.decode_frac_of_roofline",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic(w),
                     "traffic_source": f"profiles/decode_products_traffic_{w.name}.txt (FETCH_SIZE + WRITE_SIZE "
                                       "per launch of the step's products, scaled by the 1 GiB copy calibration)"
                                       if counter_traffic(w) else None,
                     "bytes_per_launch": round(step_prod_bytes / launches),
                     "avg_launch_us": round(step_prod_us / launches, 3),
                     "launches_per_step": launches,
                     "us_per_launch_by_product": {k: round(v, 3) for k, v in prod_us.items()
                                                  if k != "step_order"},
                     "bytes_per_launch_by_product": pbytes},
        "detail": {
            "gpu_event_ms_per_step": round(gpu_ms / n_steps, 3),
            "prefill_ms": round(prefill_ms, 3),
            "prefill_tok_s": round(prefill_tok_s, 1),
            "prefill_tflops": round(pf_flops / (prefill_ms / 1e3) / 1e12, 2),
            "decode_tok_s_incl_sampling": round(decode_tok_s, 2),
            "decode_step_bytes": int(step_bytes),
            "decode_roofline_tok_s": round(step_roof_tok_s, 1),
            "decode_frac_of_roofline": round(decode_tok_s / step_roof_tok_s, 4),
            "profile_ms_per_decode_step": {k: round(v, 4) for k, v in prof.items()},
            "profile_ms_per_prefill": {k: round(v, 3) for k, v in pf_prof.items()},
            "prefill_products_tflops": round(pf_gemm_tflops, 1),
            "prefill_products_frac_of_mfma": round(pf_gemm_tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "prefill_products_tflops_by_kind": {k: round(pf_gemm[k] / (pf_prof[k] / 1e3) / 1e12, 1)
                                                for k in pf_gemm},
            "create_s": round(t_create, 2),
        },
    }
    out["detail"]["prefill_rows_per_batch_row"] = T0
    h.destroy()
    del tok_dev, uni_dev, force_tok_dev, force_mask_dev
    torch.cuda.empty_cache()
    return out



if __name__ == "__main__":
    main()
