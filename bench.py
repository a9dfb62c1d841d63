#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one ``kda_chunk_prefill`` call over the whole batch of the
one-layer workload (B=1, T=8192, H=96, dk=dv=128, bf16 inputs, fp32 state,
chunk 64), inputs already resident in HBM.  ``value`` is prefill tokens/s.

The same run also times the in-place fp32 decode step (256 sequences x 96
heads, 64 consecutive steps) and reports its state bandwidth, and times the
fp64 CPU oracle on a bounded sample of the prefill workload as a baseline.

Roofline (prefill): model FLOPs per chunk-head 12C^3 + 8C^2D + 6CD^2
("Kimi K3 的架構" (hao.cnyes.com), complexity analysis of §六) over the
measured duration of the prefill launch sequence, against the bf16 dense MFMA
peak of MI355X (2.5 PFLOP/s).  Decode: 8 D^2 bytes of fp32 state per head per
token over the measured step time, against 8 TB/s HBM.
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

METRIC = "KDA prefill tokens/s (H=96,D=128) + decode state GB/s, % of MFMA/HBM peak"
C, D = 64, 128
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
FLOP_PER_CHUNK_HEAD = 12 * C ** 3 + 8 * C ** 2 * D + 6 * C * D ** 2  # 13,631,488
DECODE_BYTES_PER_HEAD_TOKEN = 8 * D * D                              # fp32 state read + write


def strip_c_comments(text: str) -> str:
    """C / C++ source without its comments and with runs of blank space
    collapsed (string and character literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: a counter summary taken on other
    code is not reported, one taken before a comment-only edit still is."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_19_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(strip_c_comments(f.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def stored_counters(workload: str):
    """SQ counter summary of the prefill call (profiles/counters_<workload>.json)
    from committed rocprofv3 runs, if they were taken on the current kernel
    sources; else None."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("call")


COPY_PROBE_FLOATS = 256 << 20   # 1 GiB fp32 read + 1 GiB written by the calibration copy
# kernels of this library, by the part of their names that identifies them
LIB_KERNELS = ("prep_kernel", "k1_kernel", "k2_kernel", "scan_kernel", "scan_bf16_kernel",
               "fused_kernel", "fused_pass1_kernel", "out_norm_gate_kernel", "decode_kernel")


def probe_dispatches(path, counters):
    """Per dispatch of a --traffic-probe counter run: (name, {counter: value})
    in dispatch order, each counter summed over its instances."""
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] not in counters:
                continue
            key = int(r["Dispatch_Id"])
            ent = rows.setdefault(key, [r["Kernel_Name"], {}])
            ent[1][r["Counter_Name"]] = ent[1].get(r["Counter_Name"], 0.0) + float(
                r["Counter_Value"])
    return [tuple(rows[k]) for k in sorted(rows)]


def probe_window(disp):
    """The measured prefill call of a --traffic-probe run: the library's
    dispatches (and the schedule uploads among them) that follow the
    calibration copy, the last call before the decode steps; and that
    copy's index."""
    first_dec = next(i for i, (n, _) in enumerate(disp) if "decode_kernel" in n)
    lib = [i for i in range(first_dec)
           if any(t in disp[i][0] for t in LIB_KERNELS)]
    i = lib[-1]
    while i >= 0 and (any(t in disp[i][0] for t in LIB_KERNELS) or "copyBuffer" in disp[i][0]):
        i -= 1
    assert i >= 0 and "elementwise" in disp[i][0].lower(), "no calibration copy before the call"
    call = [(next(t for t in LIB_KERNELS if t in n), c) for n, c in disp[i + 1:lib[-1] + 1]
            if any(t in n for t in LIB_KERNELS)]
    return i, call


def traffic_probe(kda, wl, name, dev, path="auto"):
    """One prefill call and one decode step bracketed by a plain elementwise
    copy of known size, for rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE):
    the copy's counter reading calibrates the counters to bytes."""
    import torch
    w = wl.WORKLOADS[name]
    d = wl.prefill_case(w, device=dev)
    cu = d["cu"]
    N, H = len(w.lengths), w.H
    T = int(cu[-1])
    o = torch.empty((T, H, D), dtype=w.dtype, device=dev)
    fin = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(kda.prefill_workspace_size(cu, H, w.dtype, 0, path=path), 1),
                     dtype=torch.uint8, device=dev)

    def step():
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                          initial_state=d["init"], o=o, final_state=fin, workspace=ws, path=path)

    step()                                   # warm (first-touch, schedule upload)
    torch.cuda.synchronize(dev)
    src = torch.ones(COPY_PROBE_FLOATS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    torch.mul(src, 1.0, out=dst)             # the calibration copy
    torch.cuda.synchronize(dev)
    del src, dst
    step()                                   # the measured prefill call
    torch.cuda.synchronize(dev)
    del d, o, fin, ws
    torch.cuda.empty_cache()
    wd = wl.WORKLOADS["decode_f32_N256_H96_x64"]
    dd = wl.decode_case(wd, device=dev)
    od = torch.empty((wd.lengths[0], wd.H, D), dtype=wd.dtype, device=dev)
    for _ in range(2):                       # warm, then the measured step
        kda.decode_step(dd["state"], dd["q"][0], dd["k"][0], dd["v"][0], dd["g"][0],
                        dd["beta"][0], o=od)
        torch.cuda.synchronize(dev)
    chunk_heads = sum((L + C - 1) // C for L in w.lengths) * H
    print(json.dumps({"probe": name, "copy_bytes_read": 4 * COPY_PROBE_FLOATS,
                      "copy_bytes_written": 4 * COPY_PROBE_FLOATS,
                      "chunk_heads": chunk_heads}), flush=True)


def traffic_from_counters(fetch_csv, write_csv, workload, command):
    """HBM bytes of the measured prefill call and of the decode step from two
    rocprofv3 counter files of --traffic-probe runs (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch), each scaled so that the calibration copy
    reads / writes exactly its known size."""
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "command": command, "counters": {}}
    for counter, path, known in (("FETCH_SIZE", fetch_csv, 4 * COPY_PROBE_FLOATS),
                                 ("WRITE_SIZE", write_csv, 4 * COPY_PROBE_FLOATS)):
        disp = probe_dispatches(path, (counter,))
        icopy, call = probe_window(disp)
        copy_kib = disp[icopy][1][counter]
        scale = known / (copy_kib * 1024.0)
        dec = [c[counter] for n, c in disp if "decode_kernel" in n]
        out["counters"][counter] = {
            "copy_kib": copy_kib, "scale": scale,
            "call_dispatches": [[t, c[counter] * 1024.0 * scale] for t, c in call],
            "call_bytes": sum(c[counter] for _, c in call) * 1024.0 * scale,
            "decode_bytes": dec[-1] * 1024.0 * scale if dec else None}
    f, w = out["counters"]["FETCH_SIZE"], out["counters"]["WRITE_SIZE"]
    out["hbm_bytes_per_launch"] = f["call_bytes"] + w["call_bytes"]
    if f["decode_bytes"] is not None:
        out["decode_hbm_bytes_per_step"] = f["decode_bytes"] + w["decode_bytes"]
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    with open(path, "w") as fo:
        json.dump(out, fo, indent=1)
        fo.write("\n")
    print(json.dumps(out, indent=1))


# SIMDs of one XCD: GRBM_GUI_ACTIVE counts each XCD's busy cycles, so the
# SIMD-cycles of a dispatch are this times its summed GRBM_GUI_ACTIVE
SIMDS_PER_XCD = 32 * 4


def counters_from(csv_paths, workload, command):
    """SQ activity of the measured prefill call from --traffic-probe counter
    runs (rocprofv3 --pmc, one file per pass): per dispatch and for the call,
    the fraction of SIMD cycles the MFMA unit was busy, VALU instructions per
    SIMD cycle (times 4: a wave64 VALU op holds the SIMD 4 cycles), LDS
    instructions and bank-conflict cycles per LDS-active cycle."""
    merged = None
    for path in csv_paths:
        disp = probe_dispatches(path, ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU",
                                       "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_WAVES",
                                       "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS",
                                       "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                       "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_WAIT_INST_LDS",
                                       "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"))
        _, call = probe_window(disp)
        if merged is None:
            merged = [[t, dict(c)] for t, c in call]
        else:
            assert [t for t, _ in merged] == [t for t, _ in call], "passes differ"
            for m, (_, c) in zip(merged, call):
                for k, v in c.items():
                    if k == "GRBM_GUI_ACTIVE":
                        m[1][k] = max(m[1].get(k, 0.0), v)
                    else:
                        m[1][k] = v

    def derive(c):
        simd = SIMDS_PER_XCD * c["GRBM_GUI_ACTIVE"]
        d = {"grbm_gui_active": c["GRBM_GUI_ACTIVE"]}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            d["mfma_busy_frac"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / simd
        if "SQ_INSTS_VALU" in c:
            d["valu_issue_frac"] = 4.0 * c["SQ_INSTS_VALU"] / simd
        for k in ("SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                  "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_WAVES"):
            if k in c:
                d[k.lower()] = c[k]
        if c.get("SQ_ACTIVE_INST_LDS"):
            d["lds_bank_conflict_per_active"] = (c.get("SQ_LDS_BANK_CONFLICT", 0.0) /
                                                 c["SQ_ACTIVE_INST_LDS"])
        return d

    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "command": command, "dispatches": [[t, derive(c)] for t, c in merged]}
    tot = {}
    for _, c in merged:
        for k, v in c.items():
            tot[k] = tot.get(k, 0.0) + v
    out["call"] = derive(tot)
    out["call"]["kernels"] = [t for t, _ in merged]
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % workload)
    with open(path, "w") as fo:
        json.dump(out, fo, indent=1)
        fo.write("\n")
    print(json.dumps(out, indent=1))


def time_prefill(kda, wl, name, steps, warmup, split_hint, dev, gated=False, path="auto"):
    """Event-timed prefill calls.  gated: kda_chunk_prefill_gated with every
    step on (decay gate from logits, q / k L2 norm, output norm and gate) on
    the same inputs (g serves as the gate logits, v as the output gate's)."""
    import torch
    w = wl.WORKLOADS[name]
    d = wl.prefill_case(w, device=dev)
    cu = d["cu"]
    N, H = len(w.lengths), w.H
    T = int(cu[-1])
    o = torch.empty((T, H, D), dtype=w.dtype, device=dev)
    fin = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    nbytes = kda.prefill_workspace_size(cu, H, w.dtype, split_hint, path=path)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

    A_log = torch.zeros((H,), dtype=torch.float32, device=dev)
    nw = torch.ones((D,), dtype=torch.float32, device=dev)

    def step():
        if gated:
            kda.chunk_prefill_gated(d["q"], d["k"], d["v"], d["g"], d["beta"], A_log=A_log,
                                    qk_norm_eps=1e-6, out_gate=d["v"], out_norm_weight=nw,
                                    cu_seqlens=cu, initial_state=d["init"],
                                    split_hint=split_hint, o=o, final_state=fin, workspace=ws,
                                    path=path)
        else:
            kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                              initial_state=d["init"], split_hint=split_hint, o=o,
                              final_state=fin, workspace=ws, path=path)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    ms = sum(per) / steps
    chunk_heads = sum((L + C - 1) // C for L in w.lengths) * H
    flops = chunk_heads * FLOP_PER_CHUNK_HEAD
    tflops = flops / (ms * 1e-3) / 1e12
    res = {
        "workload": name, "T": T, "H": H, "N": N, "dtype": str(w.dtype).replace("torch.", ""),
        "ms_per_step": ms, "ms_min": min(per), "wall_ms_per_step": wall / steps * 1e3,
        "tokens_per_s": T / (ms * 1e-3), "chunk_heads": chunk_heads, "model_flops": flops,
        "tflops": tflops, "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        # segments of the first sequence under this call's path (the fused
        # path takes no automatic cut; the two-kernel one the fp32 cut)
        "segments": [1 if path == "fused" and split_hint == 0 else
                     kda.plan_num_segments(L, N, H, split_hint,
                                           dtype=w.dtype if path == "auto" else None)
                     for L in w.lengths[:1]],
        "path": path,
    }
    del d, o, fin, ws
    torch.cuda.empty_cache()
    return res


def time_decode(kda, wl, dev, steps_block=64, warmup_blocks=1):
    import torch
    w = wl.WORKLOADS["decode_f32_N256_H96_x64"]
    d = wl.decode_case(w, device=dev)
    N, H = w.lengths[0], w.H
    state = d["state"]
    o = torch.empty((N, H, D), dtype=w.dtype, device=dev)

    def block():
        for s in range(w.steps):
            kda.decode_step(state, d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s],
                            o=o)

    for _ in range(warmup_blocks):
        block()
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    block()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1)
    us_step = ms * 1e3 / w.steps
    gbs = DECODE_BYTES_PER_HEAD_TOKEN * N * H / (us_step * 1e-6) / 1e9
    del d, state, o
    torch.cuda.empty_cache()
    return {"workload": w.name, "us_per_step": us_step, "state_GB_per_s": gbs,
            "hbm_frac": gbs / PEAK_HBM_GBS, "tokens_per_s": N / (us_step * 1e-6),
            "model_bytes_per_step": DECODE_BYTES_PER_HEAD_TOKEN * N * H}


def time_replay(kda, wl, dev, W=4, P=5, calls=16):
    """Speculative-decode replay at the decode workload's shape (256 sequences
    x 96 heads, fp32): W cached draft tokens, seeded accepted counts in
    [0, W], P new tokens (the bonus token and P - 1 drafts).  Next to it, the
    snapshot rollback it replaces: P single decode steps, each followed by a
    copy of the state (one snapshot per position)."""
    import numpy as np
    import torch
    w = wl.WORKLOADS["decode_f32_N256_H96_x64"]
    N, H = w.lengths[0], w.H
    c = wl.token_inputs(N * W, H, w.dtype, w.seed + 31, device=dev)
    n = wl.token_inputs(N * P, H, w.dtype, w.seed + 32, device=dev)
    cached = [c[x].reshape((N, W) + c[x].shape[1:]).contiguous() for x in ("k", "v", "g", "beta")]
    new = [n[x].reshape((N, P) + n[x].shape[1:]).contiguous()
           for x in ("q", "k", "v", "g", "beta")]
    acc_np = np.random.default_rng(w.seed + 33).integers(0, W + 1, size=N).astype(np.int32)
    acc = torch.from_numpy(acc_np).to(dev)
    state = wl.states(N, H, w.seed + 34, device=dev)
    o = torch.empty((N, P, H, D), dtype=w.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) * 1e3 / calls

    us = timed(lambda: kda.decode_replay(state, acc, *cached, *new, o=o))
    toks = [[x[:, j].contiguous() for x in new] for j in range(P)]
    snaps = [torch.empty_like(state) for _ in range(P)]
    od = torch.empty((N, H, D), dtype=w.dtype, device=dev)

    def snapshot_window():
        for j in range(P):
            kda.decode_step(state, *toks[j], o=od)
            snaps[j].copy_(state)

    us_snap = timed(snapshot_window)
    gbs = DECODE_BYTES_PER_HEAD_TOKEN * N * H / (us * 1e-6) / 1e9
    # every byte the call must move: the state read and written, the accepted
    # cached tokens' k, v, g and beta, the new tokens' q, k, v, g and beta,
    # and the new tokens' outputs
    es = torch.tensor([], dtype=w.dtype).element_size()
    token_bytes = H * es * (int(acc_np.sum()) * (3 * D + 1) + N * P * (4 * D + 1) + N * P * D)
    all_bytes = DECODE_BYTES_PER_HEAD_TOKEN * N * H + token_bytes
    del c, n, cached, new, state, o, toks, snaps
    torch.cuda.empty_cache()
    return {"shape": "N=%d H=%d fp32, W=%d cached, P=%d new" % (N, H, W, P),
            "accepted_mean": float(acc_np.mean()), "us_per_call": us,
            "state_GB_per_s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
            "bytes_per_call": all_bytes,
            "hbm_frac_all_bytes": all_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "snapshot_baseline_us": us_snap, "speedup_vs_snapshot": us_snap / us}


def copy_reference(dev, reps=5):
    """Achievable HBM bandwidth: a plain elementwise copy of 1 GiB (read 1 GiB,
    write 1 GiB), best of `reps`, as the reference next to the nominal peak."""
    import torch
    src = torch.ones(COPY_PROBE_FLOATS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize(dev)
    best = None
    stream = torch.cuda.current_stream(dev)
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.mul(src, 1.0, out=dst)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes": 8 * COPY_PROBE_FLOATS, "us": best * 1e3,
            "GB_per_s": 8 * COPY_PROBE_FLOATS / (best * 1e-3) / 1e9}


def cpu_baseline(wl, name, budget_s=10.0):
    """The fp64 oracle, as it stands, over whole heads of the workload, cycling
    through the heads until at least the time budget of compute is spent (the
    whole workload takes about a second on 16 threads, too short for a stable
    figure).  Returns tokens/s scaled to the full workload."""
    import torch
    import oracle
    w = wl.WORKLOADS[name]
    d = wl.prefill_case(w, device="cpu")
    cu = d["cu"]
    T, H = int(cu[-1]), w.H
    threads = oracle.default_threads()
    heads_done, compute_s, copy_s = 0, 0.0, 0.0
    while compute_s < budget_s:
        h0 = heads_done % H
        h1 = min(H, h0 + threads)
        t0 = time.perf_counter()
        sl = {n: d[n][:, h0:h1].double().numpy().copy()
              for n in ("q", "k", "v", "g", "beta")}
        init = None if d["init"] is None else d["init"][:, h0:h1].double().numpy()
        t1 = time.perf_counter()
        oracle.recurrence(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], cu_seqlens=cu,
                          initial_state=init, threads=threads)
        t2 = time.perf_counter()
        copy_s += t1 - t0
        compute_s += t2 - t1
        heads_done += h1 - h0
    del d
    tok_s = T * heads_done / H / compute_s
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count()
    return {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpus_allowed": allowed, "cpu_model": model,
            "sample": "%s: %d head passes (%.1f times the %d heads), all %d tokens each, fp64 "
                      "per-token recurrence; compute %.1f s (host copies %.1f s, not counted)"
                      % (name, heads_done, heads_done / H, H, T, compute_s, copy_s)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 20 untimed steps bring the device to its steady clock: with 3, a fresh
    # process times the prefill call 4-6% slower than it runs sustained
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_bf16_T8192_H96")
    ap.add_argument("--split", type=int, default=0, help="split_hint (0 = automatic)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all", action="store_true",
                    help="also time the gated call on the other workloads, and the fp32 one")
    ap.add_argument("--path", default="auto", choices=["auto", "two_kernel", "fused"],
                    help="prefill implementation (kda_prefill_options.path)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the long-context and packed-resume prefill workloads")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run one calibration copy, one prefill call and one decode step "
                         "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs) and exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two counter_collection.csv files of --traffic-probe runs into "
                         "profiles/traffic_<workload>.json (no GPU needed)")
    ap.add_argument("--counters-from", nargs="+", metavar="CSV",
                    help="turn counter_collection.csv files of --traffic-probe SQ counter runs "
                         "into profiles/counters_<workload>.json (no GPU needed)")
    ap.add_argument("--traffic-command", default="",
                    help="the command line that produced the counter files (recorded)")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from_counters(args.traffic_from[0], args.traffic_from[1], args.workload,
                              args.traffic_command)
        return
    if args.counters_from:
        counters_from(args.counters_from, args.workload, args.traffic_command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_19_amd as kda
    from gated_delta_rule_19_amd import workloads as wl

    kda.load()
    dev = torch.device("cuda:0")
    if args.traffic_probe:
        traffic_probe(kda, wl, args.workload, dev, path=args.path)
        return
    main_res = time_prefill(kda, wl, args.workload, args.steps, args.warmup, args.split, dev,
                            path=args.path)
    print("prefill %s: %.3f ms/step, %.3g tokens/s, %.1f TFLOP/s (%.1f%% of bf16 MFMA peak)"
          % (args.workload, main_res["ms_per_step"], main_res["tokens_per_s"],
             main_res["tflops"], 100 * main_res["mfma_frac"]), file=sys.stderr, flush=True)
    gated = time_prefill(kda, wl, args.workload, args.steps, args.warmup, args.split, dev,
                         gated=True, path=args.path)
    gated["vs_plain"] = gated["ms_per_step"] / main_res["ms_per_step"]
    print("prefill %s gated (decay gate, q/k norm, output norm and gate fused): %.3f ms/step "
          "(x%.3f of the plain call)" % (args.workload, gated["ms_per_step"], gated["vs_plain"]),
          file=sys.stderr, flush=True)
    # the other prefill workloads: the long-context planner and the packed
    # resume in every default run (few steps each), the gated call on them and
    # the fp32 workload with --all
    extra = {}
    names = [] if args.no_extra else ["prefill_bf16_T131072_H12",
                                      "prefill_bf16_varlen64_H96_resume"]
    if args.all:
        names.append("prefill_f32_T256_H2")
    for name in names:
        if name == args.workload:
            continue
        # as many untimed calls as the main workload's, the packed one capped
        # at 5 (about 20 ms each): with 5 the long-context call measured 5-6%
        # slower than with 20
        warm = min(args.warmup, 5) if "varlen" in name else args.warmup
        steps = 5 if "varlen" in name else max(5, args.steps // 2)
        r = time_prefill(kda, wl, name, steps, warm, 0, dev)
        r["traffic"] = stored_traffic(name)
        r["counters"] = stored_counters(name)
        extra[name] = r
        print("prefill %s: %.3f ms/step, %.3g tokens/s, %.1f%% MFMA"
              % (name, r["ms_per_step"], r["tokens_per_s"], 100 * r["mfma_frac"]),
              file=sys.stderr, flush=True)
        if args.all:
            rg = time_prefill(kda, wl, name, steps, warm, 0, dev, gated=True)
            rg["vs_plain"] = rg["ms_per_step"] / r["ms_per_step"]
            extra[name + "_gated"] = rg
            print("prefill %s gated: %.3f ms/step (x%.3f)" % (name, rg["ms_per_step"],
                                                               rg["vs_plain"]),
                  file=sys.stderr, flush=True)
    copy_ref = copy_reference(dev)
    print("plain copy: %.0f GB/s achievable (%.1f%% of the %.0f GB/s HBM peak)"
          % (copy_ref["GB_per_s"], 100 * copy_ref["GB_per_s"] / PEAK_HBM_GBS, PEAK_HBM_GBS),
          file=sys.stderr, flush=True)
    dec = None
    if not args.no_decode:
        dec = time_decode(kda, wl, dev)
        print("decode: %.1f us/step, %.0f GB/s state (%.1f%% of HBM peak)"
              % (dec["us_per_step"], dec["state_GB_per_s"], 100 * dec["hbm_frac"]),
              file=sys.stderr, flush=True)
    rep = None
    if not args.no_decode:
        rep = time_replay(kda, wl, dev)
        print("decode replay (%s, mean accepted %.2f): %.1f us/call, %.0f GB/s state (%.1f%% "
              "of HBM peak; %.1f%% with the token inputs and outputs); snapshot rollback "
              "%.1f us (x%.2f)"
              % (rep["shape"], rep["accepted_mean"], rep["us_per_call"], rep["state_GB_per_s"],
                 100 * rep["hbm_frac"], 100 * rep["hbm_frac_all_bytes"],
                 rep["snapshot_baseline_us"], rep["speedup_vs_snapshot"]),
              file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.workload)
        print("cpu oracle: %.3g tokens/s on %d threads" % (cpu["value"], cpu["cores"]),
              file=sys.stderr, flush=True)

    w = wl.WORKLOADS[args.workload]
    traffic = stored_traffic(args.workload)
    counters = stored_counters(args.workload)
    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": len(w.lengths),
                   "seq_len": int(sum(w.lengths)), "heads": w.H, "head_dim": D, "chunk": C,
                   "state": "fp32", "split_hint": args.split},
        "roofline": {"bound": "mfma", "achieved": main_res["tflops"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": main_res["mfma_frac"], "traffic": traffic,
                     "kernel": "kda_chunk_prefill call, %s implementation (%s), model "
                               "FLOPs per call / event-timed call duration"
                               % (args.path, "+".join(counters["kernels"]) if counters else
                                  "kernels per the committed counter runs"),
                     "mfma_busy_frac": counters["mfma_busy_frac"] if counters else None,
                     "valu_issue_frac": counters["valu_issue_frac"] if counters else None,
                     "hbm_GB_per_s": (traffic / (main_res["ms_per_step"] * 1e-3) / 1e9
                                      if traffic else None)},
        "hbm_reference": {"peak_GB_per_s": PEAK_HBM_GBS, "copy": copy_ref},
        "cpu_baseline": cpu,
        "prefill": main_res,
        "prefill_gated": gated,
        "decode": dec,
        "decode_replay": rep,
        "extra": extra or None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
