#!/usr/bin/env python3
"""Benchmark of the routed-MoE FFN layer on one MI355X.

One step = one pass of the whole hot path over one batch: coli_moe_route
(router GEMM, top-8, permutation) + coli_moe_ffn (grouped gate+up with the
clamped SwiGLU, grouped down, shared expert + fixed-order combine), inputs
resident in HBM.  The default workload is the T=4096 prefill batch (bf16,
Zipf-skewed router bias); the T=64 decode batch is measured as well and
reported under "decode".

Prints ONE JSON line.  Besides the throughput it reports
  roofline:     the dominant kernel (gate+up) against its bound, from HIP
                events recorded around that kernel inside the timed region;
  cpu_baseline: the CPU oracle timed on a bounded sample of the same inputs.

The default run (prefill) also measures, as extra keys of the same line: the
decode batch, the int4 workloads, the 42-layer stacked pass, the dense FFN
layers, the index top-k selection and the stacked shape with its experts
streamed through two device banks (--quick skips them).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill|decode|int4|int4_decode|stacked|tiny]
                [--tokens T] [--quick]
"""
import argparse
import csv
import ctypes as C
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA
PEAK_FP32_FLOPS = 157.3e12   # MI355X fp32 vector
PEAK_HBM = 8.0e12            # MI355X HBM3E bytes/s

WORKLOAD_NAMES = {
    "prefill": "prefill T=4096, D=2048, F=768, 288 experts top-8 + 1 shared, bf16, Zipf(1.1) router bias",
    "decode": "decode T=64, D=2048, F=768, 288 experts top-8 + 1 shared, bf16",
    "int4": "int4 experts T=512, D=2048, F=768, 288 experts top-8 + 1 shared, group 32",
    "int4_decode": "int4 experts decode T=64, D=2048, F=768, 288 experts top-8 + 1 shared, group 32",
    "tiny": "tiny T=8, D=128, F=64, 288 experts top-8 + 1 shared, fp32",
    "stacked": "stacked decode: 42 MoE layers, T=256, D=2048, F=768, 288 experts top-8 + 1 shared, "
               "bf16, fp32 residual stream",
}


# workloads around the MoE layer, measured on their own with --workload
EXTRA_WORKLOADS = ("dense_decode", "dense_prefill", "index_topk", "index_topk_decode")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# HBM traffic of the dominant kernel from rocprofv3 counters
#
# Two counter runs of the same command (FETCH_SIZE, then WRITE_SIZE; KiB per
# dispatch) are scaled by what the same counters read for a plain device copy
# of known size (--copy-calibration, 256 MiB read + 256 MiB written), and
# stored with a hash of the kernel sources.  The bench reports the traffic
# only while the sources still hash the same.
# ---------------------------------------------------------------------------
KERNEL_SOURCES = ("sparse_moe_ffn_coli_amd/csrc/ffn.hip", "sparse_moe_ffn_coli_amd/csrc/route.hip",
                  "sparse_moe_ffn_coli_amd/csrc/select.hip", "sparse_moe_ffn_coli_amd/csrc/device_common.h")
COPY_BYTES = 256 << 20


def sources_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_calibration():
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {COPY_BYTES >> 20} MiB device copy x3")


def _pmc_values(folder, counter):
    """kernel name -> list of per-dispatch counter values"""
    out = {}
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def summarize_pmc(fetch_dir, write_dir, out_path, workload, command):
    fetch, write = _pmc_values(fetch_dir, "FETCH_SIZE"), _pmc_values(write_dir, "WRITE_SIZE")
    # the calibration copies are the largest dispatches of the runtime's copy kernel
    copy = next(k for k in fetch if "copyBuffer" in k)
    f_scale = COPY_BYTES / (max(fetch[copy]) * 1024.0)
    w_scale = COPY_BYTES / (max(write[copy]) * 1024.0)
    kernels = {}
    for k, v in fetch.items():
        if not k.startswith("void coli::") and not k.startswith("coli::"):
            continue
        fk = sum(v) / len(v)
        wk = sum(write.get(k, [0.0])) / len(write.get(k, [0.0]))
        short = k.split("(")[0].replace("void ", "")
        kernels[short] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1), "dispatches": len(v),
                          "hbm_bytes": round(fk * 1024 * f_scale + wk * 1024 * w_scale)}
    summary = {"workload": workload, "command": command, "sources_sha256_16": sources_hash(),
               "copy_kernel": copy.split("(")[0], "copy_bytes_each_way": COPY_BYTES,
               "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": kernels}
    with open(out_path, "w") as f:
        json.dump(summary, f, indent=1, sort_keys=True)
    print(json.dumps(summary, indent=1, sort_keys=True))


def recorded_traffic(workload, kernel_prefix):
    """HBM bytes per launch of the kernel from the committed counter summary, or
    None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{workload}_pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        summ = json.load(f)
    if summ.get("sources_sha256_16") != sources_hash():
        return None
    for name, v in summ["kernels"].items():
        if name.split("<")[0].split("::")[-1].startswith(kernel_prefix):
            return v["hbm_bytes"]
    return None


# ---------------------------------------------------------------------------
# HIP events through the runtime's C API (recorded by the library itself on
# the stream its kernels run on)
# ---------------------------------------------------------------------------
class Hip:
    def __init__(self):
        self.L = C.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.L.hipEventSynchronize.argtypes = [C.c_void_p]
        self.L.hipEventDestroy.argtypes = [C.c_void_p]
        self.L.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            e = C.c_void_p()
            assert self.L.hipEventCreate(C.byref(e)) == 0
            out.append(e.value)
        return out

    def record(self, ev, stream):
        assert self.L.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a, b):
        ms = C.c_float()
        assert self.L.hipEventSynchronize(b) == 0
        assert self.L.hipEventElapsedTime(C.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.L.hipEventDestroy(e)


# ---------------------------------------------------------------------------
# algorithmic work of one step (per stage), from the realised routing
# ---------------------------------------------------------------------------
def algorithmic(cfg, count, int4=False):
    T, D, E, K, F = cfg["T"], cfg["D"], cfg["E"], cfg["K"], cfg["F"]
    R = T * K
    n_e = int((count > 0).sum())
    act = 4 if cfg["dtype"] == "f32" else 2              # activation / dense weight bytes
    if int4:
        G = cfg["group"]
        wbytes = lambda rows, k: rows * k // 2 + rows * (k // G) * 2
    else:
        wbytes = lambda rows, k: rows * k * act
    gu_w = n_e * 2 * wbytes(F, D) + 2 * F * D * act       # routed (non-empty) + shared gate/up
    dn_w = n_e * wbytes(D, F)
    sd_w = D * F * act
    st = {
        "router": dict(flops=2 * T * D * E, bytes=E * D * act + T * D * act + T * E * 4),
        "gate_up": dict(flops=2 * (R + T) * D * 2 * F,
                        bytes=gu_w + T * D * act + (R + T) * F * act),
        "down": dict(flops=2 * R * F * D, bytes=dn_w + R * F * act + R * D * act),
        "combine": dict(flops=2 * T * F * D + 2 * R * D,
                        bytes=sd_w + T * F * act + R * D * act + T * D * 4),
    }
    total_flops = sum(s["flops"] for s in st.values())
    # whole-step algorithmic bytes: every weight that must be read once, x in, y out
    total_bytes = (E * D * act + gu_w + dn_w + sd_w + T * D * act + T * D * 4)
    return st, total_flops, total_bytes, n_e


def roofline(flops, nbytes, seconds, peak_flops):
    t_mfma, t_hbm = flops / peak_flops, nbytes / PEAK_HBM
    if t_mfma >= t_hbm:
        a = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": peak_flops / 1e12,
                "unit": "TFLOP/s", "frac": round(a * 1e12 / peak_flops, 4)}
    a = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(a * 1e9 / PEAK_HBM, 4)}


# ---------------------------------------------------------------------------
# one workload on the GPU
# ---------------------------------------------------------------------------
def workload_inputs(name, tokens=None):
    """Config and inputs of workload ``name``; ``tokens`` overrides its batch
    size (token rows then drawn without the stored 8th/9th-gap redraws, which
    only the parity tests need)."""
    import synth

    if tokens is None:
        return synth.CONFIGS[name], synth.workload(name)
    cfg = dict(synth.CONFIGS[name], T=int(tokens))
    W = synth.layer_weights(cfg, 0)
    W["x"] = synth.x_rows(cfg, None, 0)
    return cfg, W


def run_workload(name, steps, warmup, hip, tokens=None):
    import numpy as np
    import torch

    from sparse_moe_ffn_coli_amd import COLI_BF16, COLI_F32, FFN_STAGES, ROUTE_STAGES
    from sparse_moe_ffn_coli_amd.layer import DeviceLayer, to_device

    t0 = time.time()
    cfg, W = workload_inputs(name, tokens)
    T, D, E, K, F = cfg["T"], cfg["D"], cfg["E"], cfg["K"], cfg["F"]
    log(f"{name}: generated inputs in {time.time() - t0:.1f}s")
    dt = COLI_F32 if cfg["dtype"] == "f32" else COLI_BF16
    layer = DeviceLayer(W, T, D, E, K, F, dt, group=cfg.get("group", 32))
    x = to_device(W["x"])
    del W
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream

    for _ in range(warmup):
        layer(x)
    torch.cuda.synchronize()
    log(f"{name}: {warmup} warm-up steps done")

    # per-stage breakdown (diagnostic, outside the timed region).  It runs
    # before the timed steps, which then start from a GPU in steady state
    # (clocks and caches settled by the warm-up and these steps).
    n_r, n_f = len(ROUTE_STAGES) + 1, len(FFN_STAGES) + 1
    evs = hip.events((n_r + n_f) * steps)
    for i in range(steps):
        b = evs[(n_r + n_f) * i:(n_r + n_f) * (i + 1)]
        layer(x, route_events=b[:n_r], ffn_events=b[n_r:])
    torch.cuda.synchronize()
    stage_us = {}
    for j, nm in enumerate(ROUTE_STAGES):
        stage_us[nm] = sum(hip.elapsed_ms(evs[(n_r + n_f) * i + j], evs[(n_r + n_f) * i + j + 1])
                           for i in range(steps)) / steps * 1e3
    for j, nm in enumerate(FFN_STAGES):
        o = n_r
        stage_us[nm] = sum(hip.elapsed_ms(evs[(n_r + n_f) * i + o + j],
                                          evs[(n_r + n_f) * i + o + j + 1])
                           for i in range(steps)) / steps * 1e3
    # timed region: K steps, events only at the step boundaries
    marks = hip.events(steps + 1)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    hip.record(marks[0], stream)
    for i in range(steps):
        layer(x)
        hip.record(marks[i + 1], stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    total_ms = hip.elapsed_ms(marks[0], marks[steps])
    step_ms = [hip.elapsed_ms(marks[i], marks[i + 1]) for i in range(steps)]
    log(f"{name}: {steps} timed steps, {total_ms / steps * 1e3:.1f} us/step "
        f"(host clock {host_s / steps * 1e6:.1f} us/step)")
    # the same K steps again with the library recording events around the
    # gate+up kernel of every step (ffn stage 0) on the stream it launches on:
    # the dominant kernel's duration for the roofline (recording events
    # between kernels costs a few microseconds per step, so the step time
    # above comes from the pass without them)
    gu = hip.events(2 * steps)
    marks2 = hip.events(2)
    hip.record(marks2[0], stream)
    for i in range(steps):
        layer(x, ffn_events=[gu[2 * i], gu[2 * i + 1]])
    hip.record(marks2[1], stream)
    torch.cuda.synchronize()
    instr_ms = hip.elapsed_ms(marks2[0], marks2[1])
    gu_ms = [hip.elapsed_ms(gu[2 * i], gu[2 * i + 1]) for i in range(steps)]
    log(f"{name}: instrumented pass {instr_ms / steps * 1e3:.1f} us/step, gate+up "
        f"{sum(gu_ms) / steps * 1e3:.1f} us")

    hip.destroy(gu + evs + marks + marks2)

    count = layer.routing.count.cpu().numpy()
    st, flops, nbytes, n_e = algorithmic(cfg, count, int4=cfg.get("int4", False))
    step_s = total_ms / steps / 1e3
    gu_s = sum(gu_ms) / len(gu_ms) / 1e3
    peak = PEAK_FP32_FLOPS if cfg["dtype"] == "f32" else PEAK_BF16_FLOPS
    res = dict(
        name=name, cfg=cfg, step_s=step_s, host_step_s=host_s / steps, tokens_per_s=T / step_s, n_e=n_e,
        step_median_s=float(np.median(step_ms)) / 1e3, step_min_s=min(step_ms) / 1e3,
        step_instrumented_s=instr_ms / steps / 1e3,
        flops=flops, bytes=nbytes, gu_s=gu_s, stage_us={k: round(v, 2) for k, v in stage_us.items()},
        roofline=roofline(st["gate_up"]["flops"], st["gate_up"]["bytes"], gu_s, peak),
        gate_up_work=st["gate_up"],
        mfma_pct=round(100 * flops / step_s / peak, 2),
        hbm_gbs=round(nbytes / step_s / 1e9, 1),
        hbm_pct=round(100 * nbytes / step_s / PEAK_HBM, 2),
    )
    del layer, x
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# stacked decode: 42 layers in sequence, residual add between layers
# ---------------------------------------------------------------------------
def run_stacked(steps, warmup, hip):
    import numpy as np
    import torch

    import synth
    from sparse_moe_ffn_coli_amd import COLI_BF16
    from sparse_moe_ffn_coli_amd.layer import DeviceLayer, to_device

    cfg = synth.CONFIGS["stacked"]
    T, D, E, K, F, L = cfg["T"], cfg["D"], cfg["E"], cfg["K"], cfg["F"], cfg["layers"]
    t0 = time.time()
    layers = []
    for l in range(L):
        W = synth.layer_weights(cfg, l)
        layers.append(DeviceLayer(W, T, D, E, K, F, COLI_BF16))
        del W
        if l % 6 == 5 or l == L - 1:
            log(f"stacked: {l + 1}/{L} layers generated and resident ({time.time() - t0:.0f}s)")
    x0 = to_device(synth.x_rows(cfg, synth.load_attempts("stacked"))).view(torch.bfloat16)
    xb = [torch.empty_like(x0), torch.empty_like(x0)]
    xf = torch.empty((T, D), dtype=torch.float32, device=x0.device)
    stream = torch.cuda.current_stream().cuda_stream

    def step(gu_events=None):
        # the residual stream starts from x0 every step; layer l reads bf16(x_l)
        xb[0].copy_(x0)
        xf.copy_(x0)
        cur = 0
        for l, layer in enumerate(layers):
            ev = None if gu_events is None else [gu_events[2 * l], gu_events[2 * l + 1]]
            layer(xb[cur], y=xf, residual=xf, y_bf16=xb[1 - cur], ffn_events=ev)
            cur ^= 1

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    marks = hip.events(steps + 1)
    h0 = time.perf_counter()
    hip.record(marks[0], stream)
    for i in range(steps):
        step()
        hip.record(marks[i + 1], stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    total_ms = hip.elapsed_ms(marks[0], marks[steps])
    step_ms = [hip.elapsed_ms(marks[i], marks[i + 1]) for i in range(steps)]
    gu = hip.events(2 * L * steps)                  # instrumented pass: the gate+up kernels
    for i in range(steps):
        step(gu[2 * L * i:2 * L * (i + 1)])
    torch.cuda.synchronize()
    gu_ms = [hip.elapsed_ms(gu[2 * j], gu[2 * j + 1]) for j in range(L * steps)]
    hip.destroy(gu + marks)
    step_s = total_ms / steps / 1e3
    log(f"stacked: {steps} timed steps, {step_s * 1e3:.3f} ms per 42-layer pass")

    flops = nbytes = gu_flops = gu_bytes = 0
    n_es = []
    for layer in layers:
        st, fl, nb, n_e = algorithmic(cfg, layer.routing.count.cpu().numpy())
        flops, nbytes = flops + fl, nbytes + nb
        gu_flops, gu_bytes = gu_flops + st["gate_up"]["flops"], gu_bytes + st["gate_up"]["bytes"]
        n_es.append(n_e)
    gu_s = sum(gu_ms) / len(gu_ms) / 1e3
    res = dict(name="stacked", cfg=cfg, step_s=step_s, host_step_s=host_s / steps, tokens_per_s=T / step_s,
               step_median_s=float(np.median(step_ms)) / 1e3, step_min_s=min(step_ms) / 1e3,
               step_instrumented_s=None,
               n_e=round(sum(n_es) / len(n_es), 1), flops=flops, bytes=nbytes, gu_s=gu_s,
               stage_us={}, roofline=roofline(gu_flops / L, gu_bytes / L, gu_s, PEAK_BF16_FLOPS),
               gate_up_work=dict(flops=gu_flops // L, bytes=gu_bytes // L),
               mfma_pct=round(100 * flops / step_s / PEAK_BF16_FLOPS, 2),
               hbm_gbs=round(nbytes / step_s / 1e9, 1),
               hbm_pct=round(100 * nbytes / step_s / PEAK_HBM, 2))
    del layers
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# the rows around the MoE layer: dense FFN layers, index selection, and the
# stacked workload with its experts streamed through two device banks
# ---------------------------------------------------------------------------
def _timed_calls(fn, steps, warmup, hip, stream):
    """Run fn() warmup times, then `steps` times between HIP events; returns
    the per-call durations in seconds."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    marks = hip.events(steps + 1)
    hip.record(marks[0], stream)
    for i in range(steps):
        fn()
        hip.record(marks[i + 1], stream)
    torch.cuda.synchronize()
    out = [hip.elapsed_ms(marks[i], marks[i + 1]) / 1e3 for i in range(steps)]
    hip.destroy(marks)
    return out


def _summary(times):
    import numpy as np
    return dict(mean_s=sum(times) / len(times), median_s=float(np.median(times)), min_s=min(times))


def run_dense(name, steps, warmup, hip):
    import torch

    import synth
    from sparse_moe_ffn_coli_amd import (COLI_BF16, DenseWeights, Shape, coli_moe_dense_ffn,
                                         coli_moe_dense_workspace_bytes)
    from sparse_moe_ffn_coli_amd.layer import to_device

    cfg = synth.DENSE_CONFIGS[name]
    T, D, F = cfg["T"], cfg["D"], cfg["F"]
    W = synth.dense_weights(cfg)
    shape = Shape(T, D, 0, 0, F, COLI_BF16)
    w = DenseWeights(to_device(W["gate"]), to_device(W["up"]), to_device(W["down"]))
    x = to_device(W["x"])
    ws = torch.empty(coli_moe_dense_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    t = _summary(_timed_calls(lambda: coli_moe_dense_ffn(shape, x, w, y, ws=ws), steps, warmup, hip, stream))
    flops = 2 * T * D * F * 3
    nbytes = 3 * F * D * 2 + T * D * 2 + T * D * 4
    log(f"{name}: {t['mean_s'] * 1e6:.1f} us per layer")
    return {"workload": f"dense FFN layer T={T}, D={D}, F={F}, bf16", "tokens_per_s": round(T / t["mean_s"], 1),
            "us_per_layer": round(t["mean_s"] * 1e6, 2), "us_median": round(t["median_s"] * 1e6, 2),
            "us_min": round(t["min_s"] * 1e6, 2),
            "roofline": roofline(flops, nbytes, t["mean_s"], PEAK_BF16_FLOPS),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops}


def run_index_topk(name, steps, warmup, hip):
    import torch

    import synth
    from sparse_moe_ffn_coli_amd import coli_index_topk

    cfg = synth.INDEX_CONFIGS[name]
    rows, L, k, tail = cfg["rows"], cfg["L"], cfg["k"], cfg["tail"]
    scores, lens = synth.index_scores(cfg)
    s = torch.from_numpy(scores).cuda()
    ln = torch.from_numpy(lens).cuda()
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    t = _summary(_timed_calls(lambda: coli_index_topk(s, k, idx, tail=tail, lens=ln), steps, warmup, hip, stream))
    nbytes = int(lens.astype("int64").sum()) * 4 + rows * 4 + rows * k * 4    # scores read, lens, idx written
    log(f"{name}: {t['mean_s'] * 1e6:.1f} us per call")
    return {"workload": f"index top-{k} (tail {tail}) over {rows} rows x {L} scores, fp32, "
                        f"{'causal' if cfg['lens'] == 'causal' else 'full'} lengths",
            "rows_per_s": round(rows / t["mean_s"], 1), "us_per_call": round(t["mean_s"] * 1e6, 2),
            "us_median": round(t["median_s"] * 1e6, 2), "us_min": round(t["min_s"] * 1e6, 2),
            "roofline": dict(roofline(0, nbytes, t["mean_s"], PEAK_FP32_FLOPS), algorithmic_bytes=nbytes)}


def run_bank_stream(hip, layers=4, host_layers=2):
    """The stacked decode shape with every layer's routed experts copied from
    pinned host memory into one of two device banks while the previous layer
    computes (copy stream + events).  Reports the copy alone, the compute
    alone (same layers, weights already in the banks) and the two overlapped."""
    import numpy as np
    import torch

    import synth
    from sparse_moe_ffn_coli_amd import (COLI_BF16, Routing, Shape, Weights, coli_moe_bank_acquire,
                                         coli_moe_bank_fill, coli_moe_bank_release, coli_moe_ffn,
                                         coli_moe_route, coli_moe_workspace_bytes)
    from sparse_moe_ffn_coli_amd.layer import to_device

    cfg = synth.CONFIGS["stacked"]
    T, D, E, K, F = cfg["T"], cfg["D"], cfg["E"], cfg["K"], cfg["F"]
    shape = Shape(T, D, E, K, F, COLI_BF16)
    t0 = time.time()
    host, dev = [], []
    for l in range(host_layers):
        W = synth.layer_weights(cfg, l)
        hl = []
        for k in ("gate", "up", "down"):
            a = torch.from_numpy(W[k].view(np.int16))
            p = torch.empty(a.shape, dtype=torch.int16, pin_memory=True)
            p.copy_(a)
            hl.append(p)
        host.append(hl)
        dev.append({k: to_device(W[k]) for k in ("wr", "bias", "s_gate", "s_up", "s_down")})
        del W
    log(f"bank stream: {host_layers} host layers pinned ({time.time() - t0:.0f}s)")
    banks = [[torch.empty(h.shape, dtype=torch.int16, device="cuda") for h in host[0]] for _ in range(2)]
    ready = [torch.cuda.Event() for _ in range(2)]
    free = [torch.cuda.Event() for _ in range(2)]
    copy = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    ws = torch.empty(coli_moe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    routing = Routing.empty(T, E, K)
    x = to_device(synth.x_rows(cfg, synth.load_attempts("stacked")))
    y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    layer_bytes = sum(h.numel() * 2 for h in host[0])

    def layer_compute(l):
        d, b = dev[l % host_layers], banks[l % 2]
        coli_moe_route(shape, x, d["wr"], d["bias"], routing, ws)
        coli_moe_ffn(shape, x, routing, Weights(b[0], b[1], b[2], d["s_gate"], d["s_up"], d["s_down"]), y, ws=ws)

    def fill(l, used):
        coli_moe_bank_fill(shape, host[l % host_layers], banks[l % 2], copy_stream=copy,
                           wait_event=free[l % 2] if used[l % 2] else None, ready_event=ready[l % 2])

    def streamed():
        used = [False, False]
        fill(0, used)
        for l in range(layers):
            if l + 1 < layers:
                fill(l + 1, used)
            coli_moe_bank_acquire(compute, ready[l % 2])
            layer_compute(l)
            coli_moe_bank_release(compute, free[l % 2])
            used[l % 2] = True

    def copies_only():
        for l in range(layers):
            coli_moe_bank_fill(shape, host[l % host_layers], banks[l % 2], copy_stream=copy)

    def compute_only():
        for l in range(layers):
            layer_compute(l)

    def wall(fn, reps=2):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            h = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            el = time.perf_counter() - h
            best = el if best is None else min(best, el)
        return best

    t_copy = wall(copies_only)
    t_comp = wall(compute_only)
    t_both = wall(streamed)
    # one layer's compute (copy-bound) or one layer's copy (compute-bound) cannot overlap
    ideal = max(t_copy + t_comp / layers, t_comp + t_copy / layers)
    log(f"bank stream: copy {t_copy * 1e3:.1f} ms, compute {t_comp * 1e3:.2f} ms, streamed {t_both * 1e3:.1f} ms")
    del banks, host, dev
    torch.cuda.empty_cache()
    return {"workload": f"stacked decode shape (T={T}), {layers} layers, every layer's routed experts "
                        f"({layer_bytes / 1e9:.2f} GB bf16) streamed from pinned host memory through two device banks",
            "copy_ms_per_layer": round(t_copy / layers * 1e3, 3),
            "host_to_device_gbs": round(layer_bytes * layers / t_copy / 1e9, 1),
            "compute_ms_per_layer": round(t_comp / layers * 1e3, 3),
            "streamed_ms_per_layer": round(t_both / layers * 1e3, 3),
            "tokens_per_s_streamed": round(T * layers / t_both, 1),
            "overlap_efficiency": round(ideal / t_both, 4),
            "note": "host clock around whole passes (best of 2); overlap_efficiency = ideal / streamed, ideal = "
                    "max(copies + one layer's compute, computes + one layer's copy): 1 means everything that "
                    "can overlap does"}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------
def cpu_baseline(name, budget_s=15.0, tokens=None):
    import numpy as np

    import oracle

    if name == "stacked":
        return cpu_baseline_stacked(budget_s)
    cfg, W = workload_inputs(name, tokens)
    T, D, E, K, F = cfg["T"], cfg["D"], cfg["E"], cfg["K"], cfg["F"]
    if cfg.get("int4"):
        G = cfg["group"]
        g = oracle.Mat.int4(W["gate_q"], W["gate_s"], G)
        u = oracle.Mat.int4(W["up_q"], W["up_s"], G)
        d = oracle.Mat.int4(W["down_q"], W["down_s"], G)
    else:
        g, u, d = W["gate"], W["up"], W["down"]

    def run(n):
        xs = np.ascontiguousarray(W["x"][:n])
        t = time.perf_counter()
        oracle.moe_layer(xs, W["wr"], W["bias"], g, u, d, W["s_gate"], W["s_up"], W["s_down"],
                         n, D, E, K, F)
        return time.perf_counter() - t

    threads = oracle.num_threads()
    probe = min(T, max(threads, 8))
    tp = run(probe)
    n = int(min(T, max(probe, budget_s / max(tp / probe, 1e-9))))
    n = max(probe, (n // threads) * threads) if n >= threads else n
    el = run(n) if n != probe else tp
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of the {T} tokens of the {name} workload: router over all "
                      f"{E} experts, top-{K}, routed + shared FFN, in fp64 ({el:.1f} s)"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_single_thread():
    """The oracle on one core: the tiny fp32 layer (all 8 tokens) and the
    first tokens of the decode batch."""
    import oracle

    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    out = {}
    try:
        for name, n in (("tiny", None), ("decode", 8)):
            cfg, W = workload_inputs(name)
            T, D, E, K, F = cfg["T"], cfg["D"], cfg["E"], cfg["K"], cfg["F"]
            n = T if n is None else n
            xs = W["x"][:n].copy()
            t = time.perf_counter()
            oracle.moe_layer(xs, W["wr"], W["bias"], W["gate"], W["up"], W["down"], W["s_gate"], W["s_up"],
                             W["s_down"], n, D, E, K, F)
            el = time.perf_counter() - t
            out[name] = {"tokens_per_s": round(n / el, 3), "tokens": n, "seconds": round(el, 3)}
    finally:
        oracle.set_num_threads(threads)
    return out


def cpu_baseline_stacked(budget_s):
    """The oracle's chain over the 42 layers for the first n tokens (weights
    regenerated per layer; only the oracle's own time is counted)."""
    import numpy as np

    import oracle
    import synth

    cfg = synth.CONFIGS["stacked"]
    T, D, E, K, F, L = cfg["T"], cfg["D"], cfg["E"], cfg["K"], cfg["F"], cfg["layers"]
    n = max(1, oracle.num_threads())
    x0 = synth.x_rows(cfg, synth.load_attempts("stacked"))[:n]
    x = (x0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    el = 0.0
    for l in range(L):
        W = synth.layer_weights(cfg, l)
        t = time.perf_counter()
        x = oracle.residual_layer(x, W["wr"], W["bias"], W["gate"], W["up"], W["down"],
                                  W["s_gate"], W["s_up"], W["s_down"], D, E, K, F)[5]
        el += time.perf_counter() - t
    return {"value": round(n / el, 3), "unit": "tokens/s (42-layer pass)", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"first {n} of the {T} tokens through all {L} layers in fp64 "
                                        f"({el:.1f} s of oracle time)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill",
                    choices=sorted(WORKLOAD_NAMES) + sorted(EXTRA_WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's batch size T (not for stacked)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="the named workload only (no decode, int4, stacked, dense, index or bank lines)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 256 MiB device copy first (scale for counter runs)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON"),
                    help="turn two rocprofv3 --pmc runs into a traffic summary and exit")
    ap.add_argument("--pmc-command", default="", help="command line recorded in the summary")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, workload=args.workload, command=args.pmc_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    import sparse_moe_ffn_coli_amd as pkg
    pkg.lib()
    hip = Hip()
    if args.copy_calibration:
        copy_calibration()

    if args.workload in EXTRA_WORKLOADS:
        if args.workload.startswith("dense"):
            r = run_dense(args.workload, args.steps, args.warmup, hip)
            line = {"metric": f"dense FFN tokens/s ({args.workload})", "value": r["tokens_per_s"],
                    "unit": "tokens/s", "ms_per_step": round(r["us_per_layer"] / 1e3, 5), "dtype": "bf16"}
        else:
            r = run_index_topk(args.workload, args.steps, args.warmup, hip)
            line = {"metric": f"index top-k rows/s ({args.workload})", "value": r["rows_per_s"],
                    "unit": "rows/s", "ms_per_step": round(r["us_per_call"] / 1e3, 5), "dtype": "f32"}
        line.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                     "scaling": "weak", "vs_baseline": None, "data": "synthetic (seeded generator, seed 0)",
                     "config": {"workload": r["workload"]}, "roofline": r["roofline"], "detail": r})
        print(json.dumps(line), flush=True)
        return
    if args.tokens is not None and (args.workload == "stacked" or args.tokens < 1):
        print("--tokens takes a positive batch size and a single-layer workload", file=sys.stderr)
        sys.exit(2)
    if args.workload == "stacked":
        main_res = run_stacked(args.steps, args.warmup, hip)
    else:
        main_res = run_workload(args.workload, args.steps, args.warmup, hip, args.tokens)
    full = args.workload == "prefill" and args.tokens is None and not args.quick
    dec = None
    if args.workload == "prefill" and not args.no_decode and args.tokens is None and not args.quick:
        dec = run_workload("decode", args.steps, args.warmup, hip)
    extra = {}
    if full:
        for nm in ("int4", "int4_decode"):
            extra[nm] = layer_line(run_workload(nm, args.steps, args.warmup, hip))
        extra["stacked"] = layer_line(run_stacked(max(2, args.steps // 5), 1, hip))
        extra["dense"] = {nm: run_dense(nm, args.steps, args.warmup, hip)
                          for nm in ("dense_decode", "dense_prefill")}
        extra["index_topk"] = {nm: run_index_topk(nm, args.steps, args.warmup, hip)
                               for nm in ("index_topk", "index_topk_decode")}
        extra["bank_stream"] = run_bank_stream(hip)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(args.workload, tokens=args.tokens)
        cpu["cpu_model"] = cpu_model()
        if full:
            cpu["single_thread"] = cpu_single_thread()
        log(f"cpu baseline: {cpu['value']} tokens/s on {cpu['cores']} threads")

    cfg = main_res["cfg"]
    out = {
        "metric": (f"routed-MoE tokens/s ({args.workload}, T={cfg['T']})" if args.tokens is not None else
                   "routed-MoE tokens/s at T=4096 prefill" if args.workload == "prefill" else
                   "routed-MoE tokens/s, 42-layer stacked decode (T=256)" if args.workload == "stacked"
                   else f"routed-MoE tokens/s ({args.workload})"),
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["step_s"] * 1e3, 4),
        "ms_per_step_median": round(main_res["step_median_s"] * 1e3, 4),
        "ms_per_step_min": round(main_res["step_min_s"] * 1e3, 4),
        "ms_per_step_instrumented": None if main_res.get("step_instrumented_s") is None
        else round(main_res["step_instrumented_s"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg["dtype"] == "f32" else ("fp16 (int4 weights)" if cfg.get("int4") else "bf16"),
        "data": "synthetic (seeded generator, seed 0)",
        "config": {"workload": WORKLOAD_NAMES[args.workload] + (
                       f", batch overridden to T={cfg['T']}" if args.tokens is not None else ""),
                   "global_batch": cfg["T"],
                   "seq_len": 1, "parallelism": "none (one GPU)", "experts": cfg["E"],
                   "top_k": cfg["K"], "d_model": cfg["D"], "d_ff": cfg["F"],
                   "nonempty_experts": main_res["n_e"]},
        "roofline": dict(main_res["roofline"],
                         traffic=None if args.tokens is not None else recorded_traffic(args.workload, "gateup"),
                         kernel="gate_up", avg_us=round(main_res["gu_s"] * 1e6, 2),
                         algorithmic_bytes=main_res["gate_up_work"]["bytes"],
                         algorithmic_flops=main_res["gate_up_work"]["flops"]),
        "mfma_pct": main_res["mfma_pct"],
        "hbm_gbs": main_res["hbm_gbs"],
        "hbm_pct": main_res["hbm_pct"],
        "stage_us": main_res["stage_us"],
        "cpu_baseline": cpu,
    }
    if dec is not None:
        out["decode"] = layer_line(dec)
    out.update(extra)
    print(json.dumps(out), flush=True)


def layer_line(r):
    """The extra-workload entry of the JSON line for one MoE workload result."""
    return {"workload": WORKLOAD_NAMES.get(r.get("name", ""), None) or
                        f"T={r['cfg']['T']}, D={r['cfg']['D']}, F={r['cfg']['F']}, "
                        f"{'int4 experts' if r['cfg'].get('int4') else r['cfg']['dtype']}"
                        + (f", {r['cfg']['layers']} layers" if r['cfg'].get('layers', 1) > 1 else ""),
            "tokens_per_s": round(r["tokens_per_s"], 1),
            "ms_per_step": round(r["step_s"] * 1e3, 4),
            "ms_per_step_median": round(r["step_median_s"] * 1e3, 4),
            "ms_per_step_min": round(r["step_min_s"] * 1e3, 4),
            "ms_per_step_instrumented": None if r.get("step_instrumented_s") is None
            else round(r["step_instrumented_s"] * 1e3, 4),
            "mfma_pct": r["mfma_pct"], "hbm_gbs": r["hbm_gbs"], "hbm_pct": r["hbm_pct"],
            "nonempty_experts": r["n_e"],
            "roofline": dict(r["roofline"], kernel="gate_up", avg_us=round(r["gu_s"] * 1e6, 2)),
            "stage_us": r["stage_us"]}


if __name__ == "__main__":
    main()
