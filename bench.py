"""Benchmark of the online-softmax attention hot path on one MI355X.

One step runs every kernel of the path once, each on its own workload:
  * attn_fwd, bf16, B=1, H=64, N=8192, d=128, causal, sliding window 1024,
    last 512 keys padded, 1 % of keys scaled by 8  (the headline workload);
  * attn_fwd, bf16, B=4, H=32, N=2048, d=128, causal (reported under
    `kernels`, with its fraction of the bf16 peak);
  * attn_fwd, float32, B=1, H=1, N=1000, d=64, no mask (reported under
    `kernels` in microseconds: far too small to fill the chip);
  * attn_decode_splitkv, bf16, 32 heads, 131072 keys, d=128, 64 splits;
  * online_softmax_rows, float32, 4096 x 4000;
  * online_softmax_topk_rows, float32, 1024 x 25000, k=5;
  * attn_bwd (not part of `value`): the backward pass of the headline
    workload for a seeded dO, from the O and LSE the forward wrote, counted
    at 10 d FLOPs per visible query-key pair;
  * attn_fwd_fp8 (not part of `value`): the headline workload with Q, K, V
    quantized per tensor to e4m3, against the FP8 matrix-core peak;
  * attn_fwd_exp2_offload (not part of `value`): the headline workload with
    one exponential pair in four computed on the FMA pipes.
Inputs are seeded synthetic data already resident in HBM.  Each kernel is
bracketed by HIP events on the stream it is launched on; `value` is the
forward pass's algorithmic TFLOP/s (4 d FLOPs per visible query-key pair)
over its average launch time.  Within a step the 2 GiB decode stream
evicts the softmax inputs from the caches, so those kernels read from HBM.

The `cpu_baseline` leg times the FP64 CPU oracle on this host: its top-level
figure on a bounded sample of the headline forward workload (whole heads),
and under `per_config` on a bounded sample of every other workload (whole
heads, rows or queries), about 25 s of CPU work in all.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU-oracle sample budget for the headline workload (each other workload gets a share)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three 1 GiB device-to-device copies (the reference kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(sharding across GPUs is not built)"}))
        sys.exit(2)

    import torch

    if args.copy_calibration:
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": x.numel() * 4, "copies": 3}))
        return

    import online_softmax_fa2_amd as osfa
    from online_softmax_fa2_amd import accounting as acc
    from online_softmax_fa2_amd.inputs import (WORKLOADS, attn_fp8_inputs, decode_slice, grad_inputs,
                                              softmax_rows_inputs, workload_attn_inputs)

    osfa.load_library()  # raises if the HIP library is missing
    dev = torch.device("cuda:0")

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t_setup = time.perf_counter()
    # --- forward workload -------------------------------------------------------
    fw_name = "attn_bf16_causal_w1024_pad512_b1h64_n8192_d128"
    fw = WORKLOADS[fw_name]
    fin = workload_attn_inputs(fw_name)
    fq, fk, fv = up_bf16(fin.q_bits), up_bf16(fin.k_bits), up_bf16(fin.v_bits)
    fo = torch.empty_like(fq)
    flse = torch.empty((fw["B"], fw["H"], fw["N"]), dtype=torch.float32, device=dev)
    fkv = torch.from_numpy(fin.kv_len).to(dev)
    fw_flops = acc.attn_flops(fw["B"], fw["H"], fw["N"], fw["d"], fw["causal"], fw["window"], fin.kv_len)
    # backward of the same workload
    bdo = up_bf16(grad_inputs(fw["B"], fw["H"], fw["N"], fw["d"], seed=fw["seed"])[0])
    bdq, bdk, bdv = torch.empty_like(fq), torch.empty_like(fq), torch.empty_like(fq)
    # Room to store dS: the backward forms dQ from it instead of recomputing S and dP.
    bws_bytes = max(osfa.bwd_workspace_bytes(fw["B"], fw["H"], fw["N"]),
                    osfa.bwd_stored_ds_workspace_bytes(fw["B"], fw["H"], fw["N"], fw["causal"], fw["window"]))
    bws = torch.empty((bws_bytes + 3) // 4, dtype=torch.float32, device=dev)
    bw_flops = acc.attn_bwd_flops(fw["B"], fw["H"], fw["N"], fw["d"], fw["causal"], fw["window"], fin.kv_len)
    # FP8 forward of the same workload
    f8 = attn_fp8_inputs(fw["B"], fw["H"], fw["N"], fw["d"], seed=fw["seed"], causal=fw["causal"],
                         window=fw["window"], kv_len=fw["kv_len"], n_big_keys=fw["n_big_keys"])
    f8q, f8k, f8v = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (f8.q8, f8.k8, f8.v8))
    del f8.q, f8.k, f8.v
    f8o = torch.empty_like(fo)
    f8lse = torch.empty_like(flse)
    po = torch.empty_like(fo)
    plse = torch.empty_like(flse)

    # --- causal 2048 workload and the float32 N = 1000 workload ------------------
    c3_name = "attn_bf16_causal_b4h32_n2048_d128"
    c3 = WORKLOADS[c3_name]
    c3in = workload_attn_inputs(c3_name)
    c3q, c3k, c3v = up_bf16(c3in.q_bits), up_bf16(c3in.k_bits), up_bf16(c3in.v_bits)
    c3o = torch.empty_like(c3q)
    c3lse = torch.empty((c3["B"], c3["H"], c3["N"]), dtype=torch.float32, device=dev)
    c3_flops = acc.attn_flops(c3["B"], c3["H"], c3["N"], c3["d"], c3["causal"], c3["window"], None)
    c1_name = "attn_f32_b1h1_n1000_d64"
    c1 = WORKLOADS[c1_name]
    c1in = workload_attn_inputs(c1_name)
    c1q, c1k, c1v = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (c1in.q, c1in.k, c1in.v))
    c1o = torch.empty_like(c1q)
    c1lse = torch.empty((c1["B"], c1["H"], c1["N"]), dtype=torch.float32, device=dev)
    c1_flops = acc.attn_flops(c1["B"], c1["H"], c1["N"], c1["d"], c1["causal"], c1["window"], None)

    # --- decode workload --------------------------------------------------------
    dw_name = "decode_bf16_b1h32_nkv131072_d128_split64"
    dw = WORKLOADS[dw_name]
    dq = torch.empty((dw["B"], dw["H"], dw["d"]), dtype=torch.bfloat16, device=dev)
    dk = torch.empty((dw["B"], dw["H"], dw["Nkv"], dw["d"]), dtype=torch.bfloat16, device=dev)
    dv = torch.empty_like(dk)
    for h in range(dw["H"]):
        _, _, _, qb, kb, vb = decode_slice(dw["seed"], 0, h, dw["Nkv"], dw["d"])
        dq[0, h] = up_bf16(qb)
        dk[0, h] = up_bf16(kb)
        dv[0, h] = up_bf16(vb)
    do = torch.empty((dw["B"], dw["H"], dw["d"]), dtype=torch.float32, device=dev)
    dws = torch.empty(osfa.decode_workspace_bytes(dw["B"], dw["H"], dw["d"], dw["nsplit"]) // 4,
                      dtype=torch.float32, device=dev)
    dw_bytes = acc.decode_bytes(dw["B"], dw["H"], dw["Nkv"], dw["d"])

    # --- softmax workloads ------------------------------------------------------
    sw = WORKLOADS["softmax_rows_4096x4000"]
    sx = torch.from_numpy(softmax_rows_inputs(sw["rows"], sw["cols"], seed=sw["seed"], sigma=sw["sigma"])).to(dev)
    sy = torch.empty_like(sx)
    tw = WORKLOADS["softmax_top5_1024x25000"]
    tx = torch.from_numpy(softmax_rows_inputs(tw["rows"], tw["cols"], seed=tw["seed"], sigma=tw["sigma"])).to(dev)
    tv = torch.empty((tw["rows"], tw["k"]), dtype=torch.float32, device=dev)
    ti = torch.empty((tw["rows"], tw["k"]), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    print(f"bench: inputs ready in {t_setup:.1f} s", file=sys.stderr, flush=True)

    lib = osfa.load_library()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def check(st):
        if st != 0:
            raise RuntimeError(lib.attn_last_error().decode())

    kernels = [
        ("attn_fwd", lambda: check(lib.attn_fwd(1, fq.data_ptr(), fk.data_ptr(), fv.data_ptr(), fo.data_ptr(),
                                                flse.data_ptr(), fw["B"], fw["H"], fw["N"], fw["d"], fin.scale,
                                                1, fw["window"], fkv.data_ptr(), sh))),
        ("attn_decode_splitkv", lambda: check(lib.attn_decode_splitkv(1, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                                                      do.data_ptr(), dw["B"], dw["H"], dw["Nkv"],
                                                                      dw["d"], dw["nsplit"], dws.data_ptr(),
                                                                      dws.numel() * 4, sh))),
        ("online_softmax_rows", lambda: check(lib.online_softmax_rows(sx.data_ptr(), sy.data_ptr(), sw["rows"],
                                                                      sw["cols"], sh))),
        ("online_softmax_topk_rows", lambda: check(lib.online_softmax_topk_rows(tx.data_ptr(), None, tv.data_ptr(),
                                                                                ti.data_ptr(), tw["rows"],
                                                                                tw["cols"], tw["k"], sh))),
        ("attn_fwd_fp8", lambda: check(lib.attn_fwd_fp8(f8q.data_ptr(), f8k.data_ptr(), f8v.data_ptr(),
                                                        f8o.data_ptr(), f8lse.data_ptr(), fw["B"], fw["H"], fw["N"],
                                                        fw["d"], f8.scale, f8.qd, f8.kd, f8.vd, 1, fw["window"],
                                                        fkv.data_ptr(), sh))),
        ("attn_fwd_exp2_offload", lambda: check(lib.attn_fwd_exp2_offload(
            fq.data_ptr(), fk.data_ptr(), fv.data_ptr(), po.data_ptr(), plse.data_ptr(), fw["B"], fw["H"], fw["N"],
            fw["d"], fin.scale, 1, fw["window"], fkv.data_ptr(), 4, sh))),
        ("attn_bwd", lambda: check(lib.attn_bwd(1, fq.data_ptr(), fk.data_ptr(), fv.data_ptr(), fo.data_ptr(),
                                                bdo.data_ptr(), flse.data_ptr(), bdq.data_ptr(), bdk.data_ptr(),
                                                bdv.data_ptr(), fw["B"], fw["H"], fw["N"], fw["d"], fin.scale, 1,
                                                fw["window"], fkv.data_ptr(), bws.data_ptr(), bws.numel() * 4,
                                                sh))),
        ("attn_fwd_causal_2048", lambda: check(lib.attn_fwd(1, c3q.data_ptr(), c3k.data_ptr(), c3v.data_ptr(),
                                                            c3o.data_ptr(), c3lse.data_ptr(), c3["B"], c3["H"],
                                                            c3["N"], c3["d"], c3in.scale, 1, 0, None, sh))),
        ("attn_fwd_f32_n1000", lambda: check(lib.attn_fwd(0, c1q.data_ptr(), c1k.data_ptr(), c1v.data_ptr(),
                                                          c1o.data_ptr(), c1lse.data_ptr(), c1["B"], c1["H"],
                                                          c1["N"], c1["d"], c1in.scale, 0, 0, None, sh))),
    ]

    def step(events=None):
        for i, (_, fn) in enumerate(kernels):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in kernels]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms = {name: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]))
          for i, (name, _) in enumerate(kernels)}
    ms_min = {name: float(np.min([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]))
              for i, (name, _) in enumerate(kernels)}

    fwd_tflops = fw_flops / (ms["attn_fwd"] * 1e-3) / 1e12
    dec_gbs = dw_bytes / (ms["attn_decode_splitkv"] * 1e-3) / 1e9
    sm_bytes = acc.softmax_bytes(sw["rows"], sw["cols"])
    sm_gbs = sm_bytes / (ms["online_softmax_rows"] * 1e-3) / 1e9
    tk_bytes = acc.topk_bytes(tw["rows"], tw["cols"], tw["k"])
    tk_gbs = tk_bytes / (ms["online_softmax_topk_rows"] * 1e-3) / 1e9
    bwd_tflops = bw_flops / (ms["attn_bwd"] * 1e-3) / 1e12
    f8_tflops = fw_flops / (ms["attn_fwd_fp8"] * 1e-3) / 1e12
    px_tflops = fw_flops / (ms["attn_fwd_exp2_offload"] * 1e-3) / 1e12
    c3_tflops = c3_flops / (ms["attn_fwd_causal_2048"] * 1e-3) / 1e12
    c1_tflops = c1_flops / (ms["attn_fwd_f32_n1000"] * 1e-3) / 1e12

    print(f"bench: {args.steps} timed steps done ({wall:.2f} s)", file=sys.stderr, flush=True)
    cpu = cpu_baseline(fin, fw, args.cpu_seconds)
    print("bench: CPU oracle timed on the headline workload", file=sys.stderr, flush=True)
    cpu["per_config"] = cpu_baseline_per_config(args.cpu_seconds, c1in, c3in, sx, tx, dw)

    # Measured HBM bytes per launch (rocprofv3 --pmc FETCH_SIZE + WRITE_SIZE,
    # scaled by a 1 GiB copy), recorded under profiles/ together with a hash
    # of the kernel sources: reported only while the kernel is unchanged.
    from online_softmax_fa2_amd.rocprof_summary import lookup
    traffic_file = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    fwd_grid = acc.fwd_bf16_d128_grid(fw["B"], fw["H"], fw["N"])
    fwd_traffic = lookup("fwd_bf16_d128_kernel<4, 0>", traffic_file, grid=fwd_grid)
    # Shader clock the forward kernel ran at (GRBM_GUI_ACTIVE per XCD over the
    # dispatch time, profiles/sq_counters.json): the matrix-core peak at that
    # clock is the nominal one scaled by clock / 2.4 GHz.
    sq_file = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "sq_counters.json")
    fwd_clock = lookup("fwd_bf16_d128_kernel<4, 0>", sq_file, "clock_ghz", grid=fwd_grid)
    dec_traffic = lookup("decode_partial_kernel<bf16, 128>", traffic_file)

    out = {
        "metric": "attn fwd TFLOP/s & %MFMA peak (N=8K,d=128 bf16); split-KV decode HBM GB/s",
        "value": round(fwd_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": fw_name, "B": fw["B"], "H": fw["H"], "N": fw["N"], "d": fw["d"], "causal": True,
                   "window": fw["window"], "kv_len": int(fin.kv_len[0]), "big_keys_x8": fw["n_big_keys"],
                   "algorithmic_flop": fw_flops, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": acc.PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / acc.PEAK_BF16_TFLOPS, 4),
                     "traffic": None if fwd_traffic is None else round(fwd_traffic),
                     "kernel": "fwd_bf16_d128_kernel<4, 0>", "avg_launch_us": round(ms["attn_fwd"] * 1e3, 2),
                     "clock_ghz_measured": None if fwd_clock is None else round(fwd_clock, 3),
                     "frac_at_measured_clock": None if fwd_clock is None else
                     round(fwd_tflops / (acc.PEAK_BF16_TFLOPS * fwd_clock / acc.NOMINAL_CLOCK_GHZ), 4)},
        "kernels": {
            "attn_fwd": {"workload": fw_name, "avg_us": round(ms["attn_fwd"] * 1e3, 2),
                         "min_us": round(ms_min["attn_fwd"] * 1e3, 2), "tflops": round(fwd_tflops, 2),
                         "frac_mfma_peak": round(fwd_tflops / acc.PEAK_BF16_TFLOPS, 4)},
            "attn_decode_splitkv": {"workload": dw_name, "avg_us": round(ms["attn_decode_splitkv"] * 1e3, 2),
                                    "min_us": round(ms_min["attn_decode_splitkv"] * 1e3, 2),
                                    "gbs": round(dec_gbs, 1), "frac_hbm_peak": round(dec_gbs / acc.PEAK_HBM_GBS, 4),
                                    "bytes": dw_bytes,
                                    "traffic": None if dec_traffic is None else round(dec_traffic)},
            "online_softmax_rows": {"workload": "softmax_rows_4096x4000",
                                    "avg_us": round(ms["online_softmax_rows"] * 1e3, 2),
                                    "min_us": round(ms_min["online_softmax_rows"] * 1e3, 2),
                                    "gbs": round(sm_gbs, 1), "frac_hbm_peak": round(sm_gbs / acc.PEAK_HBM_GBS, 4),
                                    "bytes": sm_bytes},
            "online_softmax_topk_rows": {"workload": "softmax_top5_1024x25000",
                                         "avg_us": round(ms["online_softmax_topk_rows"] * 1e3, 2),
                                         "min_us": round(ms_min["online_softmax_topk_rows"] * 1e3, 2),
                                         "gbs": round(tk_gbs, 1),
                                         "frac_hbm_peak": round(tk_gbs / acc.PEAK_HBM_GBS, 4), "bytes": tk_bytes},
            "attn_fwd_fp8": {"workload": fw_name + " (e4m3 Q, K, V)", "avg_us": round(ms["attn_fwd_fp8"] * 1e3, 2),
                             "min_us": round(ms_min["attn_fwd_fp8"] * 1e3, 2), "tflops": round(f8_tflops, 2),
                             "frac_mfma_peak": round(f8_tflops / acc.PEAK_FP8_TFLOPS, 4)},
            "attn_fwd_exp2_offload": {"workload": fw_name + " (1 exp pair in 4 on the FMA pipes)",
                                      "avg_us": round(ms["attn_fwd_exp2_offload"] * 1e3, 2),
                                      "min_us": round(ms_min["attn_fwd_exp2_offload"] * 1e3, 2),
                                      "tflops": round(px_tflops, 2),
                                      "frac_mfma_peak": round(px_tflops / acc.PEAK_BF16_TFLOPS, 4)},
            "attn_fwd_causal_2048": {"workload": c3_name, "avg_us": round(ms["attn_fwd_causal_2048"] * 1e3, 2),
                                     "min_us": round(ms_min["attn_fwd_causal_2048"] * 1e3, 2),
                                     "tflops": round(c3_tflops, 2),
                                     "frac_mfma_peak": round(c3_tflops / acc.PEAK_BF16_TFLOPS, 4),
                                     "algorithmic_flop": c3_flops},
            "attn_fwd_f32_n1000": {"workload": c1_name, "avg_us": round(ms["attn_fwd_f32_n1000"] * 1e3, 2),
                                   "min_us": round(ms_min["attn_fwd_f32_n1000"] * 1e3, 2),
                                   "tflops": round(c1_tflops, 3), "algorithmic_flop": c1_flops,
                                   "bound": "latency (one head of 1000 queries: 63 workgroups of 16 queries on 256 CUs)"},
            "attn_bwd": {"workload": fw_name, "avg_us": round(ms["attn_bwd"] * 1e3, 2),
                         "min_us": round(ms_min["attn_bwd"] * 1e3, 2), "tflops": round(bwd_tflops, 2),
                         "frac_mfma_peak": round(bwd_tflops / acc.PEAK_BF16_TFLOPS, 4),
                         "algorithmic_flop": bw_flops},
        },
        "cpu_baseline": cpu,
        "setup_s": round(t_setup, 1),
    }
    print(json.dumps(out), flush=True)


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(fin, fw, budget_s: float):
    """Time the FP64 oracle on whole heads of the forward workload until the budget is spent."""
    from online_softmax_fa2_amd import accounting as acc
    from oracle import attention_ref

    threads = _blas_threads()
    done = 0
    t0 = time.perf_counter()
    while done < fw["H"]:
        h = done
        attention_ref(fin.q[:, h:h + 1], fin.k[:, h:h + 1], fin.v[:, h:h + 1], fin.scale, causal=fw["causal"],
                      window=fw["window"], kv_len=fin.kv_len)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    flops = acc.attn_flops(fw["B"], done, fw["N"], fw["d"], fw["causal"], fw["window"], fin.kv_len)
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {fw['H']} heads of the forward workload (all 8192 queries each), "
                      f"FP64 NumPy oracle, {el:.1f} s"}


def cpu_baseline_per_config(budget_s: float, c1in, c3in, sx, tx, dw):
    """The FP64 oracle on a bounded sample of each other workload: whole heads (attention, decode) or whole
    rows (softmax, top-k), taken until a share of the budget is spent, scaled to the GPU metric's unit."""
    from online_softmax_fa2_amd import accounting as acc
    from online_softmax_fa2_amd.inputs import decode_slice
    from oracle import attention_ref, decode_ref, softmax_ref, topk_ref

    threads = _blas_threads()
    share = budget_s / 4.0
    out = {}

    def timed(units, run_one):
        done, t0 = 0, time.perf_counter()
        while done < units:
            run_one(done)
            done += 1
            if time.perf_counter() - t0 >= share:
                break
        return done, time.perf_counter() - t0

    # float32 attention, one head of 1000 queries: the whole workload, several times if it is quick.
    reps, el = timed(50, lambda _: attention_ref(c1in.q, c1in.k, c1in.v, c1in.scale))
    out["attn_f32_b1h1_n1000_d64"] = {"value": round(el / reps * 1e6, 1), "unit": "us", "cores": threads,
                                      "kind": "oracle", "sample": f"the whole workload, {reps} runs"}
    # bf16 causal 4 x 32 x 2048: whole heads.
    B, H, N, d = c3in.q.shape
    heads = [(b, h) for b in range(B) for h in range(H)]
    n, el = timed(len(heads), lambda i: attention_ref(
        c3in.q[heads[i][0]:heads[i][0] + 1, heads[i][1]:heads[i][1] + 1],
        c3in.k[heads[i][0]:heads[i][0] + 1, heads[i][1]:heads[i][1] + 1],
        c3in.v[heads[i][0]:heads[i][0] + 1, heads[i][1]:heads[i][1] + 1], c3in.scale, causal=True))
    fl = acc.attn_flops(1, n, N, d, True, 0, None)
    out["attn_bf16_causal_b4h32_n2048_d128"] = {"value": round(fl / el / 1e12, 6), "unit": "TFLOP/s",
                                                "cores": threads, "kind": "oracle",
                                                "sample": f"{n} of {len(heads)} heads, {el:.1f} s"}
    # row softmax and the fused top-5: blocks of 64 whole rows.
    xs = sx.cpu().numpy()
    n, el = timed(xs.shape[0] // 64, lambda i: softmax_ref(xs[64 * i:64 * i + 64]))
    out["softmax_rows_4096x4000"] = {"value": round(acc.softmax_bytes(64 * n, xs.shape[1]) / el / 1e9, 3),
                                     "unit": "GB/s", "cores": threads, "kind": "oracle",
                                     "sample": f"{64 * n} of {xs.shape[0]} rows, {el:.1f} s"}
    xt = tx.cpu().numpy()
    n, el = timed(xt.shape[0] // 16, lambda i: topk_ref(xt[16 * i:16 * i + 16], 5))
    out["softmax_top5_1024x25000"] = {"value": round(acc.topk_bytes(16 * n, xt.shape[1], 5) / el / 1e9, 3),
                                      "unit": "GB/s", "cores": threads, "kind": "oracle",
                                      "sample": f"{16 * n} of {xt.shape[0]} rows, {el:.1f} s"}
    # split-KV decode: whole heads (the oracle needs no split).
    def dec(h):
        q, k, v, _, _, _ = decode_slice(dw["seed"], 0, h, dw["Nkv"], dw["d"])
        t = time.perf_counter()
        decode_ref(q[None, None], k[None, None], v[None, None])
        return time.perf_counter() - t
    spent, n, t0 = 0.0, 0, time.perf_counter()
    while n < dw["H"] and time.perf_counter() - t0 < share:  # the budget covers input generation too
        spent += dec(n)
        n += 1
    out["decode_bf16_b1h32_nkv131072_d128_split64"] = {
        "value": round(acc.decode_bytes(1, n, dw["Nkv"], dw["d"]) / spent / 1e9, 3), "unit": "GB/s",
        "cores": threads, "kind": "oracle",
        "sample": f"{n} of {dw['H']} heads (input generation not timed), {spent:.1f} s"}
    return out


if __name__ == "__main__":
    main()
