"""Throughput of the fused MXFP8 QKV path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input already resident in
HBM: residual add + RMSNorm + ROW_MX quantisation of the bf16 hidden states, the ROW_MX x MX
FP8 QKV projection with its fused dequant / bias / sum-of-squares epilogue, and the in-place
across-heads RMSNorm + 3-axis rotate-half RoPE on Q and K.  Workload: the full video shape,
T = 75600 tokens (21 x 45 x 80 grid), H = 5120, 40 Q + 40 KV heads x 128 (I = 15360).

Prints ONE JSON line.  ``value`` is the projection's algorithmic TFLOP/s over the whole step
(2 * T * H * I / step time).  Per-kernel durations come from HIP events recorded on the stream
the library launches on, averaged over the timed steps.  ``configs`` times every other workload
in the same run (the tiny, moderate and full-video self-attention projections with their norm +
RoPE pass, the moderate one also with a 2 GiB last-level-cache flush between steps, and the
cross-attention's three separate projections).  ``cpu_baseline`` times the CPU oracle (NumPy,
fp64) on a bounded row sample of the same workload on this host.  The SHA-256 prefix of every
generated input buffer is part of ``config``.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5|3|2] [--act rowmx|mx] [--headnorm none|rms|ln]
                    [--layout bsd|nbsd] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QKV proj TFLOP/s (% MXFP8 MFMA peak) + norm/RoPE GB/s, S=75600 H=5120"
PEAK_MXFP8_TFLOPS = 5000.0          # MI355X dense MXFP8 MFMA
PEAK_HBM_GBS = 8000.0               # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "project_kernel_c5_traffic.json")
PROJECT_SRC = [os.path.join(ROOT, "rope_mxfp8_qkv_amd", "csrc", f)
               for f in ("project_kernel.h", "project.hip")]


def source_digest(paths) -> str:
    """sha256 prefix of the projection's sources (the kernel header and its ROW_MX launcher)."""
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernels):
    """HBM bytes per projection call (the sum over `kernels`, the kernels the call launches)
    from the committed counter summary, or None when the kernel source changed since the
    counters were taken or a kernel is missing from it."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("kernel_src_sha256_16") != source_digest(PROJECT_SRC):
        return None
    per = rec.get("per_kernel", {})
    if any(k not in per for k in kernels):
        return None
    return sum(per[k]["read_bytes"] + per[k]["write_bytes"] for k in kernels)


def copy_calibration(nbytes: int):
    """A plain device-to-device copy of a known size (torch's copy kernel), run a few times."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}), flush=True)


def power_phases(secs: float):
    """Back-to-back calls, `secs` seconds each: the staged projection at the full video shape on
    the workload's codes, the same call on all-zero activation and weight codes, then the MFMA
    rate probe on random and on zero register operands.  Prints one JSON line per phase start
    and end (wall-clock seconds) so that board power and clocks sampled by another process
    (`amd-smi metric -p -c --json` in a loop) can be assigned to the phases; the end line also
    gives the mean time per call."""
    import torch
    import rope_mxfp8_qkv_amd as q
    dev = torch.device("cuda:0")
    inp = gen_inputs(5, dev)
    p = inp["p"]
    T, H, I = p.T, p.H, p.I
    codes = torch.empty((H // 4, I, 4), dtype=torch.uint8, device=dev)
    e8 = torch.empty((H // 32, I), dtype=torch.uint8, device=dev)
    q.mx_weight_quantize(inp["w"], codes, e8)
    wp = q.prepare_weight(codes, e8, H, I)
    wz = q.prepare_weight(torch.zeros_like(codes), e8, H, I)
    img = torch.empty(q.qkv_act_image_bytes(T, H), dtype=torch.uint8, device=dev)
    sc = torch.empty((T,), dtype=torch.float32, device=dev)
    res_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_quantize_staged(inp["hid"], inp["pgamma"], 1e-6, img, sc, residual=inp["res"],
                                 residual_out=res_out)
    zimg = torch.zeros_like(img)
    out = torch.empty((T, I), dtype=torch.bfloat16, device=dev)
    ssq = torch.empty((T, 2), dtype=torch.float32, device=dev)
    ws = torch.empty(q.qkv_staged_workspace_bytes(T, I), dtype=torch.uint8, device=dev)
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clocks = torch.empty((blocks, 2), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def proj(im, w):
        q.qkv_rowmx_project_staged(im, sc, w, out, H=H, num_heads=p.num_heads,
                                   num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                                   bias=inp["bias"], ssq=ssq, workspace=ws)

    def phase(name, fn, per_sync):
        t0 = time.time()
        print(json.dumps({"phase": name, "start": t0}), flush=True)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        n = 0
        while time.time() - t0 < secs:
            for _ in range(per_sync):
                fn()
                n += 1
            torch.cuda.synchronize()
        b.record(stream)
        torch.cuda.synchronize()
        print(json.dumps({"phase": name, "end": time.time(), "calls": n,
                          "ms_per_call": a.elapsed_time(b) / n}), flush=True)

    t0 = time.time()
    time.sleep(min(secs, 3.0))
    print(json.dumps({"phase": "idle", "start": t0, "end": time.time()}), flush=True)
    phase("projection_workload_codes", lambda: proj(img, wp), 5)
    phase("projection_zero_codes", lambda: proj(zimg, wz), 5)
    phase("mfma_probe_random", lambda: q.mfma_rate_probe(blocks, 20000, True, sink, clocks), 2)
    phase("mfma_probe_zero", lambda: q.mfma_rate_probe(blocks, 20000, False, sink, clocks), 2)


def summarize_power(phases_log: str, samples_file: str, skip_s: float = 1.0):
    """Mean board power and graphics clock per phase (CPU only) from power_phases' JSON lines and
    a file of `T <unix time>` lines each followed by one `amd-smi metric -p -c --json` output;
    the first `skip_s` seconds of each phase are left out (the clock settles)."""
    import re
    txt = open(samples_file).read()
    parts = re.split(r"^T (\d+\.\d+)\n", txt, flags=re.M)
    samples = []
    for i in range(1, len(parts), 2):
        body = parts[i + 1]
        try:
            j = json.loads(body[:body.rfind("}") + 1])
        except ValueError:
            continue
        g = j["gpu_data"][0] if isinstance(j, dict) else j[0]
        gfx = [v["clk"]["value"] for k, v in g["clock"].items()
               if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
               and isinstance(v["clk"].get("value"), (int, float))]
        samples.append((float(parts[i]), float(g["power"]["socket_power"]["value"]),
                        sum(gfx) / len(gfx) if gfx else float("nan")))
    ph = {}
    for line in open(phases_log):
        if line.startswith("{"):
            d = json.loads(line)
            ph.setdefault(d["phase"], {}).update(d)
    out = []
    for name, d in ph.items():
        sel = [x for x in samples if d["start"] + skip_s <= x[0] <= d["end"]]
        if not sel:
            continue
        out.append({"phase": name, "samples": len(sel),
                    "power_w": sum(x[1] for x in sel) / len(sel),
                    "power_w_min": min(x[1] for x in sel), "power_w_max": max(x[1] for x in sel),
                    "gfx_clock_mhz": sum(x[2] for x in sel) / len(sel),
                    "ms_per_call": d.get("ms_per_call")})
    for o in out:
        print(json.dumps(o))
    return out


PROJECTION_KERNELS = ("act_repack_kernel", "project_kernel", "ssq_reduce_kernel")
STAGED_KERNELS = ("project_kernel", "ssq_reduce_kernel")   # + a 1-block counter reset


def _counter_means(run_dir: str, counter: str):
    """Mean value of `counter` per dispatch, per kernel name, from a rocprofv3 --pmc CSV run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    acc = {}
    for f in files:
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"].replace("(anonymous namespace)::", "")
            name = name.split("(")[0].split("<")[0].split("::")[-1].split()[-1]
            key = (name, row["Dispatch_Id"])
            acc[key] = acc.get(key, 0.0) + float(row["Counter_Value"])
    per = {}
    for (name, _), v in acc.items():
        per.setdefault(name, []).append(v)
    return {k: sum(v) / len(v) for k, v in per.items()}


def summarize_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes):
    """Scaled HBM bytes per projection call from four rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE of the benchmark, the same two of a plain copy of copy_bytes bytes, which give
    the counters' scale), written to the traffic record the benchmark line reports."""
    import synth
    p = synth.CONFIGS[5].calls[0]
    copy_kib = copy_bytes / 1024.0
    cf = _counter_means(copy_fetch_dir, "FETCH_SIZE")
    cw = _counter_means(copy_write_dir, "WRITE_SIZE")
    ck = max(cf, key=cf.get)                       # the copy kernel: the largest dispatch
    fetch_scale, write_scale = copy_kib / cf[ck], copy_kib / cw[ck]
    fk, wk = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    T, H, I = p.T, p.H, p.I
    alg = {"act_repack_kernel": (T * H, T * H),
           "project_kernel": (T * H + H * I + T * 4, 2 * T * I),
           "ssq_reduce_kernel": (4 * T * 2 * ((p.Iq + p.Ik) // 128), 8 * T)}
    per = {}
    for k in PROJECTION_KERNELS:
        if k not in fk or k not in wk:
            continue
        per[k] = {"fetch_kib": fk[k], "write_kib": wk[k],
                  "read_bytes": fk[k] * 1024 * fetch_scale, "write_bytes": wk[k] * 1024 * write_scale,
                  "alg_read_bytes": alg[k][0], "alg_write_bytes": alg[k][1]}
    # the step's two HBM-bound kernels, for comparison with their algorithmic bytes (not part
    # of the projection call's traffic)
    Iqk = p.Iq + p.Ik
    other_alg = {"rmsnorm_quantize_wave_kernel": (4 * T * H + 2 * H, 2 * T * H + T * (H + 4)),
                 "norm_rope_kernel": (2 * T * Iqk + 8 * T * p.head_dim + 8 * T + 2 * Iqk,
                                      2 * T * Iqk)}
    others = {}
    for k, (ar, aw) in other_alg.items():
        if k in fk and k in wk:
            others[k] = {"fetch_kib": fk[k], "write_kib": wk[k],
                         "read_bytes": fk[k] * 1024 * fetch_scale,
                         "write_bytes": wk[k] * 1024 * write_scale,
                         "alg_read_bytes": ar, "alg_write_bytes": aw}
    rec = {"what": f"HBM bytes per dispatch of the projection's kernels ({', '.join(per)}) at "
                   f"T={T} H={H} I={I}, from rocprofv3 FETCH_SIZE/WRITE_SIZE scaled by a "
                   f"{copy_bytes}-byte copy calibration (copy kernel {ck})",
           "kernel_src_sha256_16": source_digest(PROJECT_SRC),
           "fetch_scale": fetch_scale, "write_scale": write_scale, "per_kernel": per,
           "hbm_bytes_per_call": sum(v["read_bytes"] + v["write_bytes"] for v in per.values()),
           "other_step_kernels": others}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"traffic_file": TRAFFIC_FILE, "hbm_bytes_per_call": rec["hbm_bytes_per_call"],
                      "fetch_scale": fetch_scale, "write_scale": write_scale}))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="5: producer + self-attention projection at the full video shape (the "
                         "headline); 3 / 2 / 1: the self-attention projection at T = 75600 / "
                         "4096 / 128 (activations quantised once, outside the step); 4: the "
                         "cross-attention's three separate projections (Q from 75600 latent "
                         "tokens, K and V from 512 context tokens) with the norm on Q and K")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the MFMA-rate and copy-bandwidth calibration after the timed steps")
    ap.add_argument("--layout", choices=["bsd", "nbsd"], default="bsd",
                    help="output layout of the projection and pass 2 (BSD [T, I] or NBSd [I/d, T, d])")
    ap.add_argument("--act-layout", choices=["staged", "packed"], default="staged",
                    help="activation hand-over between producer and projection: codes (and MX "
                         "exponents) written by the producer in the projection's operand layout, "
                         "ROW_MX scales as an fp32 array (staged), or the pages' row layouts "
                         "([T, H + 4] ROW_MX rows; [T, H] codes + [T, H / 32] exponents) re-laid "
                         "by the projection on every call (packed)")
    ap.add_argument("--act", choices=["rowmx", "mx"], default="rowmx",
                    help="activation encoding: ROW_MX rows with an fp32 row scale (the projection's "
                         "packed_hidden) or MX block-32 (E8M0 exponent per 32 elements)")
    ap.add_argument("--headnorm", choices=["none", "rms", "ln"], default="none",
                    help="per-head qk-norm (RMS_NORM / LAYER_NORM) + RoPE fused into the projection's "
                         "epilogue instead of the across-heads norm pass (ROW_MX activations)")
    ap.add_argument("--cpu-rows", type=int, default=16384)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the block that times every other workload (C1-C4, C2 also with a "
                         "MALL flush) after the headline run")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step into a HIP graph and time --steps replays of it "
                         "(stages.graph_ms_per_step)")
    ap.add_argument("--flush-mall", type=int, default=0, metavar="BYTES",
                    help="write a BYTES-byte scratch buffer between timed steps (outside the step's "
                         "events) so that no step finds the previous step's data in the 256 MB "
                         "last-level cache; ms_per_step is then the mean of the steps' own events")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                                                             "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="only write the traffic record from four rocprofv3 --pmc runs (no GPU)")
    ap.add_argument("--power-phases", type=float, default=0.0, metavar="SECONDS",
                    help="only run back-to-back projection calls (workload codes, then zero codes) "
                         "and MFMA probe calls (random, then zero operands), SECONDS each, printing "
                         "wall-clock phase markers for an outside power / clock sampler")
    ap.add_argument("--summarize-power", nargs=2, metavar=("PHASES_LOG", "SAMPLES"),
                    help="only print mean board power and clock per phase (no GPU)")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30,
                    help="size of the calibration copy the --summarize-traffic runs used")
    return ap.parse_args()


def gen_inputs(cid, dev):
    import torch

    import synth
    cfg = synth.CONFIGS[cid]
    p = cfg.calls[0]
    t0 = time.time()

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def dv(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    inp = {"p": p, "producer": cfg.producer}
    digests = {}

    def keep(name, a):                 # SHA-256 prefix of every generated host buffer
        digests[name] = synth.digest(a)
        return a

    if cfg.producer:
        hid, res, gam = synth.producer_inputs(cid, p.T, p.H)
        inp.update(hid=bf(keep("hidden", hid)), res=bf(keep("residual", res)),
                   pgamma=bf(keep("producer_gamma", gam)))
        del hid, res
    else:
        inp["x"] = dv(keep("activation", synth.activation(p)))
    inp["w"] = dv(keep("weight", synth.weight(p)))
    inp["bias"] = bf(keep("bias", synth.bias_bf16(p)))
    inp["gq"] = bf(keep("q_gamma", synth.gamma_bf16(p, "q")))
    inp["gk"] = bf(keep("k_gamma", synth.gamma_bf16(p, "k")))
    cos, sin = synth.rope_tables(p)
    inp["cos"], inp["sin"] = dv(keep("cos", cos)), dv(keep("sin", sin))
    inp["gen_s"] = time.time() - t0
    inp["sha256"] = digests
    return inp


def algorithmic_bytes(p, producer: bool, mx: bool = False):
    """Per-kernel algorithmic HBM bytes (each input read once, each output written once)."""
    T, H, Iq, Ik, d = p.T, p.H, p.Iq, p.Ik, p.head_dim
    nr = 4 * T * (Iq + Ik) + (8 * T * d if p.rope else 0) + 8 * T + 2 * (Iq + Ik)
    # producer: hidden + residual in, residual sum out, encoded rows out (ROW_MX: H codes + fp32
    # scale; MX: H codes + H / 32 exponents), gamma once
    enc = T * (H + H // 32) if mx else T * (H + 4)
    prod = 4 * T * H + 2 * T * H + enc + 2 * H if producer else 0
    return {"norm_rope": nr, "producer": prod}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def synth_configs_separate(cid: int) -> bool:
    """Whether workload `cid` is made of several separate projection calls."""
    import synth
    return len(synth.CONFIGS[cid].calls) > 1


def stage_stats(ms, names):
    """Median and minimum over the timed steps of each stage's event time (ms)."""
    return {n: {"median": float(np.median(ms[:, i])), "min": float(ms[:, i].min())}
            for i, n in enumerate(names)}


def run_gpu(args):
    import torch

    import rope_mxfp8_qkv_amd as q
    dev = torch.device("cuda:0")
    log(f"generating inputs for config {args.config}")
    inp = gen_inputs(args.config, dev)
    log(f"inputs ready in {inp['gen_s']:.1f} s")
    p = inp["p"]
    T, H, I = p.T, p.H, p.I
    stream = torch.cuda.current_stream()

    # weight preparation (one-time, untimed)
    codes = torch.empty((H // 4, I, 4), dtype=torch.uint8, device=dev)
    e8 = torch.empty((H // 32, I), dtype=torch.uint8, device=dev)
    q.mx_weight_quantize(inp["w"], codes, e8)
    wp = q.prepare_weight(codes, e8, H, I)
    del inp["w"], codes, e8

    mx = args.act == "mx"
    hn = {"none": 0, "rms": q.HEAD_RMS_NORM, "ln": q.HEAD_LAYER_NORM}[args.headnorm]
    if hn and mx:
        raise SystemExit("--headnorm runs on ROW_MX activations")
    if hn:     # per-head gammas / beta: the first head_dim entries of the seeded segment draws
        d = p.head_dim
        hgq, hgk = inp["gq"][:d].contiguous(), inp["gk"][:d].contiguous()
        hbq = (inp["bias"][:d].contiguous() if hn == q.HEAD_LAYER_NORM else None)
        hbk = (inp["bias"][d:2 * d].contiguous() if hn == q.HEAD_LAYER_NORM else None)
    if mx and args.act_layout == "packed":
        codes_a = torch.empty((T, H), dtype=torch.uint8, device=dev)
        e8_a = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    staged = args.act_layout == "staged"
    if staged:
        img = torch.empty(q.qkv_act_image_bytes(T, H), dtype=torch.uint8, device=dev)
        if mx:
            eimg = torch.empty(q.qkv_act_exp_image_bytes(T, H) // 4, dtype=torch.int32, device=dev)
        else:
            row_scale = torch.empty((T,), dtype=torch.float32, device=dev)
    elif not mx:
        packed = torch.empty((T, H + 4), dtype=torch.uint8, device=dev)
    res_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if inp["producer"] else None
    layout = q.LAYOUT_NBSD if args.layout == "nbsd" else q.LAYOUT_BSD
    out = (torch.empty((I // p.head_dim, T, p.head_dim), dtype=torch.bfloat16, device=dev)
           if args.layout == "nbsd" else torch.empty((T, I), dtype=torch.bfloat16, device=dev))
    ssq = torch.empty((T, 2), dtype=torch.float32, device=dev)
    ws_n = (q.qkv_staged_workspace_bytes(T, I) if staged else
            q.qkv_mx_workspace_bytes(T, H, I) if mx else q.qkvmx_workspace_bytes(T, H, I))
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    flags = q.NORM_Q | q.NORM_K | q.FUSED_ROPE
    if not inp["producer"]:                         # activations fixed for the whole run
        if mx and staged:
            q.mx_block_quantize_staged(inp["x"], img, eimg)
        elif mx:
            q.mx_block_quantize(inp["x"], codes_a, e8_a)
        elif staged:
            q.row_quantize_staged(inp["x"], img, row_scale)
        else:
            q.row_quantize_packed(inp["x"], packed)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        if inp["producer"]:
            if mx and staged:
                q.rmsnorm_mx_block_quantize_staged(inp["hid"], inp["pgamma"], 1e-6, img, eimg,
                                                   residual=inp["res"], residual_out=res_out)
            elif mx:
                q.rmsnorm_mx_block_quantize(inp["hid"], inp["pgamma"], 1e-6, codes_a, e8_a,
                                            residual=inp["res"], residual_out=res_out)
            elif staged:
                q.rmsnorm_mx_quantize_staged(inp["hid"], inp["pgamma"], 1e-6, img, row_scale,
                                             residual=inp["res"], residual_out=res_out)
            else:
                q.rmsnorm_mx_quantize(inp["hid"], inp["pgamma"], 1e-6, packed,
                                      residual=inp["res"], residual_out=res_out)
        if ev:
            ev[1].record(stream)
        if hn:
            hkw = dict(H=H, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                       head_dim=p.head_dim, norm_kind=hn, q_gamma=hgq, k_gamma=hgk, q_beta=hbq,
                       k_beta=hbk, eps=1e-6, cos=inp["cos"], sin=inp["sin"], bias=inp["bias"],
                       workspace=ws, layout=layout)
            if staged:
                q.qkv_rowmx_project_headnorm_staged(img, row_scale, wp, out, **hkw)
            else:
                q.qkv_rowmx_project_headnorm(packed, wp, out, **hkw)
        elif mx and staged:
            q.qkv_mx_project_staged(img, eimg, wp, out, T=T, H=H, num_heads=p.num_heads,
                                    num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                                    bias=inp["bias"], ssq=ssq, workspace=ws, layout=layout)
        elif staged:
            q.qkv_rowmx_project_staged(img, row_scale, wp, out, H=H, num_heads=p.num_heads,
                                       num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                                       bias=inp["bias"], ssq=ssq, workspace=ws, layout=layout)
        elif mx:
            q.qkv_mx_project(codes_a, e8_a, wp, out, H=H, num_heads=p.num_heads,
                             num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, bias=inp["bias"],
                             ssq=ssq, workspace=ws, layout=layout)
        else:
            q.qkv_rowmx_project(packed, wp, out, H=H, num_heads=p.num_heads,
                                num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
                                bias=inp["bias"], ssq=ssq, workspace=ws, layout=layout)
        if ev:
            ev[2].record(stream)
        if not hn:
            q.qk_norm_rope_apply(out, num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                 head_dim=p.head_dim, eps=1e-6, flags=flags, ssq=ssq,
                                 q_gamma=inp["gq"], k_gamma=inp["gk"], cos=inp["cos"],
                                 sin=inp["sin"], layout=layout)
        if ev:
            ev[3].record(stream)

    flush = (torch.empty(args.flush_mall // 4, dtype=torch.float32, device=dev)
             if args.flush_mall else None)
    for k in range(args.warmup):
        if flush is not None:
            flush.fill_(float(k))
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps"
        + (f", {args.flush_mall} bytes written between steps" if flush is not None else ""))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush.fill_(float(k))
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                      for e in evs])
    ms = stage.mean(axis=0)          # producer, projection (+ sum reduce), norm/rope
    graph_ms = None
    if args.graph:                   # the same step as one HIP graph, replayed back to back
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t1) * 1e3 / args.steps
        log(f"graph replays: {graph_ms:.4f} ms/step")
    ms_step = (float(stage.sum(axis=1).mean()) if flush is not None else wall * 1e3 / args.steps)
    flops = 2.0 * T * H * I
    nbytes = algorithmic_bytes(p, inp["producer"], mx)
    proj_tflops = flops / (ms[1] * 1e-3) / 1e12
    res = {
        "ms_per_step": ms_step,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "stage_ms": {"producer": float(ms[0]), "projection": float(ms[1]),
                     "norm_rope": float(ms[2])},
        "stage_stats": stage_stats(stage, ["producer", "projection", "norm_rope"]),
        "graph_ms_per_step": graph_ms,
        "projection_tflops": proj_tflops,
        "norm_rope_gbs": None if hn else nbytes["norm_rope"] / (ms[2] * 1e-3) / 1e9,
        "producer_gbs": (nbytes["producer"] / (ms[0] * 1e-3) / 1e9) if inp["producer"] else None,
        "flops": flops,
        "bytes": nbytes,
        "gen_s": inp["gen_s"],
        "sha256": inp["sha256"],
        "p": p,
        "producer": inp["producer"],
        "mx": mx,
        "staged": staged,
        "headnorm": args.headnorm,
    }
    return res


def measure_ceilings(p=None):
    """What this GPU sustains outside the kernels, measured in the same run (context for the
    roofline fractions, which divide by the published peaks): the scaled FP8 MFMA issue rate on
    register operands (random E4M3 codes, as the workload's, and zeros) with the clock the chip
    held meanwhile, the bandwidth of a plain device-to-device copy (read + write bytes) and, for
    the projection's shape ``p``, torch's FP8 GEMM with one scale per tensor (the vendor
    library's kernel; no block scales, no sum of squares) on random E4M3 operands."""
    import torch
    import rope_mxfp8_qkv_amd as q
    dev = torch.device("cuda:0")
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 20000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clocks = torch.empty((blocks, 2), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    res = {}
    for rnd in (True, False):
        best = None
        for _ in range(4):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            q.mfma_rate_probe(blocks, iters, rnd, sink, clocks)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            c = clocks.cpu().numpy().astype(np.float64)
            ghz = float(np.mean(c[:, 0] / (c[:, 1] / 100e6)) / 1e9)
            tf = blocks * 4 * iters * 16 * 131072.0 / (ms * 1e-3) / 1e12
            if best is None or tf > best[0]:
                best = (tf, ghz)
        key = "random" if rnd else "zero"
        res[f"mfma_{key}_operands_tflops"] = best[0]
        res[f"mfma_{key}_operands_clock_ghz"] = best[1]
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    ts = []
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    res["hbm_copy_gbs"] = 2.0 * n / (float(np.median(ts[1:])) * 1e-3) / 1e9
    res["mfma_probe"] = (f"{blocks} blocks x 4 wavefronts x {iters} x 16 "
                         "V_MFMA_SCALE_F32_32X32X64_F8F6F4 on register operands, best of 4")
    res["copy"] = f"torch device copy of {n} bytes, median of 5"
    del src, dst
    if p is not None:
        res.update(library_gemm(p.T, p.H, p.I))
    return res


def library_gemm(M, K, N):
    """torch._scaled_mm (tensor-wise scales) at [M, K] x [K, N] -> bf16: codes spread over the
    E4M3 range as the workload's (|x| up to 448), median of 10 timed calls after 3 warm-ups."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    a = torch.randn(M, K, device=dev, generator=g).mul_(100.0).clamp_(-448, 448).to(torch.float8_e4m3fn)
    b = torch.randn(N, K, device=dev, generator=g).mul_(150.0).clamp_(-448, 448).to(torch.float8_e4m3fn)
    sa = torch.tensor(1.0 / 100, device=dev)
    sb = torch.tensor(1.0 / 150, device=dev)
    stream = torch.cuda.current_stream()
    ts = []
    for i in range(13):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        out = torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            ts.append(e0.elapsed_time(e1))
        del out
    ms = float(np.median(ts))
    return {"library_fp8_gemm_ms": ms,
            "library_fp8_gemm_tflops": 2.0 * M * K * N / (ms * 1e-3) / 1e12,
            "library_fp8_gemm": (f"torch._scaled_mm, tensor-wise scales, [{M}, {K}] x [{K}, {N}] "
                                 "e4m3 -> bf16, median of 10")}


def run_gpu_separate(args):
    """The cross-attention workload: three single-segment projections (num_kv_heads = 0) on
    staged ROW_MX activations, each followed by its norm pass where the call norms (no RoPE).
    The activations are quantised once, outside the timed step."""
    import torch

    import rope_mxfp8_qkv_amd as q
    import synth
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    stream = torch.cuda.current_stream()
    t0 = time.time()
    calls = []
    for p in cfg.calls:
        c = {"p": p}
        x = torch.from_numpy(synth.activation(p)).to(dev)
        c["img"] = torch.empty(q.qkv_act_image_bytes(p.T, p.H), dtype=torch.uint8, device=dev)
        c["sc"] = torch.empty((p.T,), dtype=torch.float32, device=dev)
        q.row_quantize_staged(x, c["img"], c["sc"])
        del x
        w = torch.from_numpy(synth.weight(p)).to(dev)
        codes = torch.empty((p.H // 4, p.I, 4), dtype=torch.uint8, device=dev)
        e8 = torch.empty((p.H // 32, p.I), dtype=torch.uint8, device=dev)
        q.mx_weight_quantize(w, codes, e8)
        c["wp"] = q.prepare_weight(codes, e8, p.H, p.I)
        del w, codes, e8
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        c["bias"] = bf(synth.bias_bf16(p))
        c["gq"] = bf(synth.gamma_bf16(p, "q"))
        c["out"] = torch.empty((p.T, p.I), dtype=torch.bfloat16, device=dev)
        c["flags"] = (q.NORM_Q if p.norm_q else 0) | (q.FUSED_ROPE if p.rope else 0)
        c["ssq"] = torch.empty((p.T, 2), dtype=torch.float32, device=dev) if c["flags"] & q.NORM_Q else None
        c["ws"] = torch.empty(q.qkv_staged_workspace_bytes(p.T, p.I), dtype=torch.uint8, device=dev)
        calls.append(c)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    def step(ev=None):
        for i, c in enumerate(calls):
            p = c["p"]
            if ev:
                ev[2 * i].record(stream)
            q.qkv_rowmx_project_staged(c["img"], c["sc"], c["wp"], c["out"], H=p.H,
                                       num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                       head_dim=p.head_dim, bias=c["bias"], ssq=c["ssq"],
                                       workspace=c["ws"])
            if ev:
                ev[2 * i + 1].record(stream)
            if c["flags"]:
                q.qk_norm_rope_apply(c["out"], num_heads=p.num_heads, num_kv_heads=p.num_kv_heads,
                                     head_dim=p.head_dim, eps=1e-6, flags=c["flags"], ssq=c["ssq"],
                                     q_gamma=c["gq"])
        if ev:
            ev[-1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_ev = 2 * len(calls) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = [c["p"].name for c in calls]
    proj = np.array([[e[2 * i].elapsed_time(e[2 * i + 1]) for i in range(len(calls))] for e in evs])
    after = np.array([[e[2 * i + 1].elapsed_time(e[2 * i + 2]) for i in range(len(calls))] for e in evs])
    ms_step = wall * 1e3 / args.steps
    flops = [2.0 * c["p"].T * c["p"].H * c["p"].I for c in calls]
    stages, rates = {}, {}
    stats = {**stage_stats(proj, [f"{n}_projection" for n in names]),
             **stage_stats(after, [f"{n}_after_projection" for n in names])}
    for i, c in enumerate(calls):
        p = c["p"]
        pm = float(proj[:, i].mean())
        stages[f"{names[i]}_projection"] = pm
        rates[f"{names[i]}_projection_tflops"] = flops[i] / (pm * 1e-3) / 1e12
        if c["flags"]:
            nm = float(after[:, i].mean())
            nbytes = 4 * p.T * p.Iq + 8 * p.T + 2 * p.Iq
            stages[f"{names[i]}_norm"] = nm
            rates[f"{names[i]}_norm_gbs"] = nbytes / (nm * 1e-3) / 1e9
    big = int(np.argmax(flops))
    ach = rates[f"{names[big]}_projection_tflops"]
    line = {
        "metric": METRIC, "value": sum(flops) / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8 (e4m3 x e4m3 -> fp32 MFMA), fp32 norm, bf16 I/O", "data": "synthetic",
        "config": {"workload": "cross-attention: separate Q, K, V projections on staged ROW_MX "
                               "activations + across-heads norm on Q and K (no RoPE)",
                   "calls": [{"name": c["p"].name, "T": c["p"].T, "H": c["p"].H, "I": c["p"].I}
                             for c in calls],
                   "parallelism": "single GPU"},
        "roofline": {"kernel": f"qkv_rowmx_project_staged ({names[big]} call)", "bound": "mfma",
                     "achieved": ach, "peak": PEAK_MXFP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_MXFP8_TFLOPS, "traffic": None},
        "stages": {"ms": stages, "ms_median_min": stats, **rates},
        "ceilings": None, "cpu_baseline": None,
    }
    return line


def _compact(r):
    """The per-workload figures of one run_gpu result."""
    p = r["p"]
    d = {"T": p.T, "H": p.H, "I": p.I,
         "step_ms": r["ms_per_step"],
         "projection_ms": r["stage_ms"]["projection"],
         "projection_tflops": r["projection_tflops"],
         "projection_frac_of_peak": r["projection_tflops"] / PEAK_MXFP8_TFLOPS,
         "norm_rope_ms": r["stage_ms"]["norm_rope"],
         "norm_rope_gbs": r["norm_rope_gbs"],
         "norm_rope_hbm_frac": (r["norm_rope_gbs"] / PEAK_HBM_GBS) if r["norm_rope_gbs"] else None}
    return d


def run_config_block(args):
    """Every other workload, measured in the same run with the same library calls as their own
    ``--config N`` runs: the tiny (C1), moderate (C2) and full-video (C3) self-attention
    projections with the norm + RoPE pass (activations quantised once, outside the step), C2
    again with a 2 GiB scratch write between steps (so no step finds the previous one's data
    in the 256 MB last-level cache), and the cross-attention's three separate projections (C4)."""
    steps, warm = max(5, min(args.steps, 10)), 2
    block = {}
    for cid, flush in ((1, 0), (2, 0), (2, 2 << 30), (3, 0)):
        a = argparse.Namespace(**vars(args))
        a.config, a.steps, a.warmup, a.flush_mall, a.graph = cid, steps, warm, flush, False
        r = _compact(run_gpu(a))
        if flush:
            block["C2"]["with_mall_flush_2GiB"] = r
        else:
            block[f"C{cid}"] = r
        log(f"config block: C{cid}{' (MALL flush)' if flush else ''}: projection "
            f"{r['projection_tflops']:.0f} TFLOP/s, norm {r['norm_rope_gbs']:.0f} GB/s")
    a = argparse.Namespace(**vars(args))
    a.config, a.steps, a.warmup = 4, steps, warm
    line = run_gpu_separate(a)
    st = line["stages"]
    block["C4"] = {"step_ms": line["ms_per_step"], "calls": line["config"]["calls"],
                   "ms": st["ms"],
                   **{k: v for k, v in st.items() if k.endswith("_tflops") or k.endswith("_gbs")},
                   **{k[:-len("_tflops")] + "_frac_of_peak": v / PEAK_MXFP8_TFLOPS
                      for k, v in st.items() if k.endswith("_projection_tflops")},
                   **{k[:-len("_gbs")] + "_hbm_frac": v / PEAK_HBM_GBS
                      for k, v in st.items() if k.endswith("_norm_gbs")}}
    block["note"] = (f"{steps} timed steps after {warm} warm-ups per workload; projection = the "
                     "staged ROW_MX call (counter reset + project_kernel + sum reduce), norm = "
                     "the norm (+ RoPE) pass, each timed with HIP events on the library's stream")
    return block


def cpu_baseline(cid, rows_n):
    """The oracle, as it stands, on the first ``rows_n`` tokens of the same workload."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas_pools] or [1])
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in blas_pools) or None
    except Exception:                                        # pragma: no cover
        threads, blas = 1, None
    cfg = synth.CONFIGS[cid]
    p = cfg.calls[0]
    rows = np.arange(rows_n)
    w = synth.weight(p)
    if cfg.producer:
        hid, res, gam = synth.producer_inputs(cid, p.T, p.H, row_idx=rows)
    else:
        x = synth.activation(p, row_idx=rows)
    cos, sin = synth.rope_tables(p, rows)
    bias, gq, gk = synth.bias_bf16(p), synth.gamma_bf16(p, "q"), synth.gamma_bf16(p, "k")
    wc, we = oracle.mx_weight_quantize(w)                   # weight prep: untimed, as on the GPU
    t0 = time.perf_counter()
    if cfg.producer:
        _, packed, _ = oracle.rmsnorm_rowmx(hid, res, gam, 1e-6)
    else:
        packed = oracle.rowmx_quantize(x)
    t1 = time.perf_counter()
    codes, sA = oracle.rowmx_unpack(packed, p.H)
    X, ssq = oracle.project(codes, sA, wc, we, None, bias, num_heads=p.num_heads,
                            num_kv_heads=p.num_kv_heads, head_dim=p.head_dim)
    xb = oracle.f64_to_bf16(X)
    t2 = time.perf_counter()
    oracle.norm_rope(xb, ssq, gq, gk, cos, sin, num_heads=p.num_heads,
                     num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, eps=1e-6, flags=7)
    t3 = time.perf_counter()
    dt = t3 - t0
    flops = 2.0 * rows_n * p.H * p.I
    nb = algorithmic_bytes(dataclasses.replace(p, T=rows_n), cfg.producer)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "cores_note": "BLAS threads of the fp64 contraction (the oracle's only threaded "
                          "stage; the rest runs on one core)",
            "host_cores_available": len(os.sched_getaffinity(0)),
            "kind": "oracle", "blas": blas,
            "stages": {"producer_or_quantise_s": t1 - t0,
                       "producer_gbs": (nb["producer"] / (t1 - t0) / 1e9) if cfg.producer else None,
                       "projection_s": t2 - t1, "projection_tflops": flops / (t2 - t1) / 1e12,
                       "norm_rope_s": t3 - t2, "norm_rope_gbs": nb["norm_rope"] / (t3 - t2) / 1e9},
            "sample": f"first {rows_n} of {p.T} tokens, whole step (producer/quantise, "
                      f"fp64 projection incl. weight decode, norm+RoPE); {dt:.1f} s"}


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.copy_bytes)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.summarize_power:
        summarize_power(*args.summarize_power)
        return
    if args.power_phases:
        power_phases(args.power_phases)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU; --gpus must be 1 "
                                   "(the path shards by tokens with no exchange; multi-GPU runs "
                                   "are not part of this benchmark)"}))
        sys.exit(2)
    if synth_configs_separate(args.config):
        print(json.dumps(run_gpu_separate(args)), flush=True)
        return
    r = run_gpu(args)
    p = r["p"]
    log(f"gpu: {r['ms_per_step']:.3f} ms/step, stages {r['stage_ms']}")
    ceil = None if args.no_ceilings else measure_ceilings(p)
    if ceil:
        ceil["projection_frac_of_mfma_random"] = r["projection_tflops"] / ceil["mfma_random_operands_tflops"]
        ceil["projection_vs_library_fp8_gemm"] = r["projection_tflops"] / ceil["library_fp8_gemm_tflops"]
        if r["norm_rope_gbs"]:
            ceil["norm_rope_frac_of_copy"] = r["norm_rope_gbs"] / ceil["hbm_copy_gbs"]
        if r["producer_gbs"]:
            ceil["producer_frac_of_copy"] = r["producer_gbs"] / ceil["hbm_copy_gbs"]
        log(f"ceilings: {ceil}")
    block = None
    if not args.no_configs and args.config == 5 and args.layout == "bsd" and not r["mx"] \
            and r["headnorm"] == "none" and r["staged"]:
        block = run_config_block(args)
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_rows} rows")
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.config, args.cpu_rows)
    ach = r["projection_tflops"]
    line = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 (e4m3 x e4m3 -> fp32 MFMA), fp32 norm/RoPE, bf16 I/O",
        "data": "synthetic",
        "config": {
            "workload": (("producer + QKV projection with per-head %s + 3-axis RoPE fused"
                          % {"rms": "RMS_NORM", "ln": "LAYER_NORM"}[r["headnorm"]])
                         if r["headnorm"] != "none" else
                         ("producer + QKV projection + across-heads norm + 3-axis RoPE"
                          if r["producer"] else "QKV projection + across-heads norm + RoPE"))
                        + (", MX block-32 activations" if r["mx"] else ", ROW_MX activations")
                        + (" staged in the projection's operand layout" if r["staged"] else
                           " as natural-order codes and exponents" if r["mx"] else
                           " as packed [T, H+4] rows"),
            "T": p.T, "H": p.H, "I": p.I, "num_heads": p.num_heads,
            "num_kv_heads": p.num_kv_heads, "head_dim": p.head_dim,
            "grid": list(p.grid) if p.grid else None, "layout": args.layout.upper().replace("NBSD", "NBSd"),
            "parallelism": "single GPU",
            "mall_flush_bytes_between_steps": args.flush_mall,
            "inputs_sha256_16": r["sha256"],
        },
        "roofline": {
            "kernel": ("qkv_mx_project_staged (counter reset + project_kernel + ssq_reduce)"
                       if r["mx"] and r["staged"] else
                       "qkv_mx_project (activation repacks + project_kernel + ssq_reduce)"
                       if r["mx"] else
                       ("qkv_rowmx_project_headnorm_staged (counter reset + project_kernel)"
                        if r["staged"] else
                        "qkv_rowmx_project_headnorm (activation repack + project_kernel)")
                       if r["headnorm"] != "none" else
                       "qkv_rowmx_project_staged (counter reset + project_kernel + ssq_reduce)"
                       if r["staged"] else
                       "qkv_rowmx_project (activation repack + project_kernel + ssq_reduce)"),
            "bound": "mfma",
            "achieved": ach,
            "peak": PEAK_MXFP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": ach / PEAK_MXFP8_TFLOPS,
            "traffic": (measured_traffic(STAGED_KERNELS if r["staged"] else PROJECTION_KERNELS)
                        if args.config == 5 and args.layout == "bsd" and not r["mx"]
                        and r["headnorm"] == "none" else None),
        },
        "stages": {
            "ms": r["stage_ms"],
            "ms_median_min": r["stage_stats"],
            "graph_ms_per_step": r["graph_ms_per_step"],
            "projection_tflops": r["projection_tflops"],
            "norm_rope_gbs": r["norm_rope_gbs"],
            "norm_rope_hbm_frac": (r["norm_rope_gbs"] / PEAK_HBM_GBS) if r["norm_rope_gbs"] else None,
            "producer_gbs": r["producer_gbs"],
            "producer_hbm_frac": (r["producer_gbs"] / PEAK_HBM_GBS) if r["producer_gbs"] else None,
        },
        "ceilings": ceil,
        "configs": block,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
