"""Benchmark of the online-softmax attention hot path on one MI355X.

One step runs every kernel of the path once, each on its own workload:
  * attn_fwd, bf16, B=1, H=64, N=8192, d=128, causal, sliding window 1024,
    last 512 keys padded, 1 % of keys scaled by 8  (the headline workload);
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

The `cpu_baseline` leg times the FP64 CPU oracle on a bounded sample of the
forward workload (whole heads, about 15 s of CPU work) on this host.

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
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-oracle sample budget")
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
    bws = torch.empty(osfa.bwd_workspace_bytes(fw["B"], fw["H"], fw["N"]) // 4, dtype=torch.float32, device=dev)
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

    cpu = cpu_baseline(fin, fw, args.cpu_seconds)

    # Measured HBM bytes per launch (rocprofv3 --pmc FETCH_SIZE + WRITE_SIZE,
    # scaled by a 1 GiB copy), recorded under profiles/ together with a hash
    # of the kernel sources: reported only while the kernel is unchanged.
    from online_softmax_fa2_amd.rocprof_summary import lookup
    traffic_file = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    fwd_traffic = lookup("fwd_bf16_d128_kernel<4, 0>", traffic_file)
    # Shader clock the forward kernel ran at (GRBM_GUI_ACTIVE per XCD over the
    # dispatch time, profiles/sq_counters.json): the matrix-core peak at that
    # clock is the nominal one scaled by clock / 2.4 GHz.
    sq_file = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "sq_counters.json")
    fwd_clock = lookup("fwd_bf16_d128_kernel<4, 0>", sq_file, "clock_ghz")
    dec_traffic = lookup("decode_partial_kernel", traffic_file)

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
            "attn_bwd": {"workload": fw_name, "avg_us": round(ms["attn_bwd"] * 1e3, 2),
                         "min_us": round(ms_min["attn_bwd"] * 1e3, 2), "tflops": round(bwd_tflops, 2),
                         "frac_mfma_peak": round(bwd_tflops / acc.PEAK_BF16_TFLOPS, 4),
                         "algorithmic_flop": bw_flops},
        },
        "cpu_baseline": cpu,
        "setup_s": round(t_setup, 1),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(fin, fw, budget_s: float):
    """Time the FP64 oracle on whole heads of the forward workload until the budget is spent."""
    from online_softmax_fa2_amd import accounting as acc
    from oracle import attention_ref

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
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


if __name__ == "__main__":
    main()
