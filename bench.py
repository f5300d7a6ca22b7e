"""Benchmark: jagged attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1] [--no-cpu-baseline]

A step is one pass of the whole hot path (forward, then the backward's Di,
dK/dV and dQ stages, or the fused block kernels) over one batch of seeded
synthetic inputs that are resident in HBM before timing starts.  The value is
fwd+bwd TFLOP/s counted over valid (unpadded) tokens only:
    FLOPs_fwd = 4 H D sum_b lq_b lk_b        FLOPs_bwd = 2.5 FLOPs_fwd
Every launch is also timed with HIP events on the stream it runs on; the
kernel with the largest share gets a roofline entry.  The fp64 CPU oracle is
timed beside it on a bounded sample of the same workload (first samples in
order, fwd+bwd) as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_FP8_TFLOPS = 5033.2   # dense MXFP8 / FP8 MFMA: twice the bf16 rate
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


WARM_S = 0.5  # seconds of back-to-back untimed steps before the timed region


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=1, help="workload index 0..8 (1 = headline)")
    ap.add_argument("--order", default="zigzag", help="unit order across workers (the zigzag deal by default)")
    ap.add_argument("--workers", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-mib", type=int, default=1024, help="copy size of the counter calibration")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (counter calibration) and exit")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="write profiles/mfma.json for --config from a rocprofv3 MFMA counter run in DIR")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "CALIB_FETCH", "CALIB_WRITE"),
                    help="turn four rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE of this workload; "
                         "the same two of --copy-calib) into profiles/traffic.json and exit")
    return ap.parse_args()


def copy_calibration(mib, steps):
    """Plain device copy of a known size: the reference point that scales the
    FETCH_SIZE / WRITE_SIZE counters of the attention kernels to bytes."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.randn(n, device="cuda")
    y = torch.empty_like(x)
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": steps}))


def rowstats_in_dq(w):
    """Whether the library's dQ pass forms Di and LSE*log2e itself (bf16
    softmax without the block mask, except D = 128 with fp32 O): then
    there is no separate Di pass, and dQ runs before dK/dV."""
    return (w.act == "softmax" and not w.block_diagonal and not w.mxfp8 and w.dtype == "bf16"
            and not (w.D == 128 and w.out_dtype == "f32"))


def kernel_work(w, info, es_in, es_out, es_g, es_db=4, mx=None):
    """Algorithmic bytes and FLOPs of each launch (every interface tensor once)."""
    H, D = w.H, w.D
    Tq, Tk, nb = int(info.Tq), int(info.Tk), int(info.bias_elems)
    qd, kd = Tq * H * D, Tk * H * D
    F = float(info.flops_fwd)
    bias_in = nb * es_in if w.bias else 0
    dbias_out = nb * es_db if w.want_dbias else 0
    rowstat = Tq * H * 4
    if w.block_diagonal:
        return {
            "block_fwd": (3 * qd * es_in + qd * es_out, F),
            "block_bwd": (4 * qd * es_in + 3 * qd * es_g, 2.5 * F),
        }
    if w.mxfp8:
        # codes 1 byte per element; the transposed copies ~1 byte per element
        # (plus the zero tails of partial 32-token blocks); scales 1/32 byte
        nq, nk = mx  # (codes, codes_t, scales) bytes of a query-row and a key-row tensor
        return {
            "quant": (2 * (2 * qd + 2 * kd) + 2 * sum(nq) + 2 * sum(nk), 0.0),
            "fwd": (nq[0] + nq[2] + nk[0] + nk[1] + 2 * nk[2] + qd * es_out + rowstat, F),
            "prep": (nq[0] + nq[2] + qd * es_out + rowstat + 2 * rowstat, 2.0 * qd),
            "dkdv": (2 * sum(nq) + nk[0] + nk[0] + 2 * nk[2] + 2 * rowstat + 2 * kd * es_g, 2.0 * F),
            "dq": (2 * (nq[0] + nq[2]) + sum(nk) + nk[0] + nk[2] + 2 * rowstat + qd * es_g, 0.5 * F),
        }
    soft = w.act == "softmax"
    work = {
        "fwd": (qd * es_in + 2 * kd * es_in + bias_in + qd * es_out + (rowstat if soft else 0), F),
        "dkdv": (2 * qd * es_in + 2 * kd * es_in + bias_in + (2 * rowstat if soft else 0)
                 + 2 * kd * es_g + dbias_out, 2.0 * F),
        "dq": (2 * qd * es_in + 2 * kd * es_in + bias_in + (2 * rowstat if soft else 0) + qd * es_g, 0.5 * F),
    }
    if soft and rowstats_in_dq(w):
        # dQ also reads O and LSE and writes Di and LSE*log2e (instead of reading them)
        b_, f_ = work["dq"]
        work["dq"] = (b_ + qd * es_out + rowstat, f_ + 2.0 * qd)
    elif soft:
        work["prep"] = (qd * es_out + qd * es_in + rowstat, 2.0 * qd)
    if w.qk_norm:
        # read Q and K, write their normalised copies and 1/||row||; the
        # backward reads Q, K and the gradients of the copies, writes dQ, dK
        work["qknorm"] = (2 * (qd + kd) * es_in + (Tq + Tk) * H * 4, 3.0 * (qd + kd))
        work["qknorm_bwd"] = ((qd + kd) * es_in + 2 * (qd + kd) * es_g, 6.0 * (qd + kd))
    return work


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "jagged_variable_length_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


KERNEL_KEYS = [("mx_quant_kernel", "quant"), ("block_fwd_kernel", "block_fwd"), ("block_bwd_kernel", "block_bwd"), ("dkdv", "dkdv"),
               ("dq2_kernel", "dq"), ("dq_kernel", "dq"), ("fwd2_kernel", "fwd"), ("fwd_kernel", "fwd"),
               ("di_kernel", "prep"), ("l2norm_fwd_kernel", "qknorm"), ("l2norm_bwd_kernel", "qknorm_bwd")]


def kernel_key(name):
    """Launch name used in the bench line for a (mangled) kernel name."""
    for pat, key in KERNEL_KEYS:
        if pat in name:
            return key
    return None


def traffic_for(kernel, cfg):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources and this workload (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    ent = d.get("workloads", {}).get(str(cfg), {}).get(kernel)
    return ent.get("bytes_per_launch") if ent else None


def _pmc_means(folder, counter):
    """Mean value of `counter` per dispatch, by kernel name, from the
    *counter_collection.csv files rocprofv3 wrote under `folder`."""
    import csv
    per = {}
    for root, _, files in os.walk(folder):
        for f in files:
            if not f.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(root, f)) as fh:
                for row in csv.DictReader(fh):
                    if row.get("Counter_Name") != counter:
                        continue
                    key = (row["Kernel_Name"], row.get("Dispatch_Id", ""))
                    per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {n: (float(np.mean(v)), len(v)) for n, v in out.items()}


def traffic_summary(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each attention kernel,
    scaled by what the same counters read for a plain copy of known size."""
    fetch, write, cfetch, cwrite = args.traffic_summary
    calib_bytes = args.calib_mib * (1 << 20)
    cf_ = max(_pmc_means(cfetch, "FETCH_SIZE").items(), key=lambda kv: kv[1][1])
    cw_ = max(_pmc_means(cwrite, "WRITE_SIZE").items(), key=lambda kv: kv[1][1])
    f_read = calib_bytes / (cf_[1][0] * 1024.0)
    f_write = calib_bytes / (cw_[1][0] * 1024.0)
    res = {}
    fm, wm = _pmc_means(fetch, "FETCH_SIZE"), _pmc_means(write, "WRITE_SIZE")
    for name, (kib, n) in fm.items():
        key = kernel_key(name)
        if key is None:
            continue
        wkib = wm.get(name, (0.0, 0))[0]
        rd, wr = kib * 1024.0 * f_read, wkib * 1024.0 * f_write
        res[key] = {"kernel": name, "dispatches": n, "fetch_kib": kib, "write_kib": wkib,
                    "read_bytes": rd, "write_bytes": wr, "bytes_per_launch": rd + wr}
    out = {"source_hash": source_hash(), "calibration": {
        "copy_bytes": calib_bytes, "copy_kernel": cf_[0], "fetch_kib": cf_[1][0], "write_kib": cw_[1][0],
        "read_factor": f_read, "write_factor": f_write}, "workloads": {str(args.config): res}}
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(p):
        try:
            old = json.load(open(p))
        except (OSError, ValueError):
            old = {}
        if old.get("source_hash") == out["source_hash"]:
            old.get("workloads", {}).update(out["workloads"])
            out["workloads"] = old["workloads"]
    with open(p, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def _pmc_rows(folder):
    """Rows of the *counter_collection.csv files rocprofv3 wrote under `folder`."""
    import csv
    for root, _, files in os.walk(folder):
        for f in files:
            if f.endswith("counter_collection.csv"):
                with open(os.path.join(root, f)) as fh:
                    yield from csv.DictReader(fh)


def mfma_summary(args):
    """MFMA utilisation and shader clock of each attention kernel from one
    rocprofv3 run with --pmc MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
    SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8.

    MfmaUtil = 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max over XCDs of
    GRBM_GUI_ACTIVE * 1024 SIMDs), rocprofiler's own definition; the csv
    carries GRBM_GUI_ACTIVE summed over the XCDs, so the per-XCD maximum is
    recovered from that definition, and the clock is that many cycles over the
    dispatch's duration (a lower bound: the duration includes launch edges).
    MOPS counters give the MFMA work actually executed (x 512 FLOP)."""
    per = {}
    for row in _pmc_rows(args.mfma_summary):
        key = (row["Kernel_Name"], row["Dispatch_Id"])
        d = per.setdefault(key, {"ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"])})
        d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    by = {}
    for (name, _), d in per.items():
        by.setdefault(name, []).append(d)
    res = {}
    for name, ds in by.items():
        key = kernel_key(name)
        if key is None:
            continue
        m = lambda c: float(np.mean([d.get(c, 0.0) for d in ds]))
        util, busy, ns = m("MfmaUtil"), m("SQ_VALU_MFMA_BUSY_CYCLES"), m("ns")
        gui_max = busy * 100.0 / (util * 1024) if util > 0 else None
        res[key] = {"kernel": name, "dispatches": len(ds), "mfma_util_pct": round(util, 2),
                    "mfma_busy_cycles": busy, "grbm_gui_active_sum": m("GRBM_GUI_ACTIVE"),
                    "grbm_gui_active_max_xcd": gui_max, "duration_us": round(ns / 1e3, 2),
                    "clock_mhz": round(gui_max / ns * 1e3, 0) if gui_max else None,
                    "mfma_flops_bf16": m("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512,
                    "mfma_flops_f8": m("SQ_INSTS_VALU_MFMA_MOPS_F8") * 512}
    out = {"source_hash": source_hash(), "workloads": {str(args.config): res}}
    p = os.path.join(ROOT, "profiles", "mfma.json")
    if os.path.exists(p):
        try:
            old = json.load(open(p))
        except (OSError, ValueError):
            old = {}
        if old.get("source_hash") == out["source_hash"]:
            old.get("workloads", {}).update(out["workloads"])
            out["workloads"] = old["workloads"]
    with open(p, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def mfma_for(kernel, cfg):
    """Counter record of `kernel` on workload `cfg` (profiles/mfma.json), if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "mfma.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    return d.get("workloads", {}).get(str(cfg), {}).get(kernel)


def _window_pairs(n, window):
    left, right = window
    return sum(min(n - 1, i + right) - max(0, i - left) + 1 for i in range(n))


def host_info():
    """(BLAS threads, {cpu model, BLAS vendor and version, usable cores}) of
    the process running the oracle."""
    cores, host = None, {}
    try:
        from threadpoolctl import threadpool_info
        blas = [t for t in threadpool_info() if t.get("user_api") == "blas"]
        cores = max([t.get("num_threads", 1) for t in blas] or [1])
        if blas:
            host["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    host["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        host["usable_cores"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return cores, host


class ClockSampler:
    """Samples the shader clock the amdgpu kernel driver reports (the active level of
    pp_dpm_sclk of the card in use) while the timed steps run."""

    def __init__(self, torch):
        self.path, self.samples, self._stop = None, [], False
        try:
            bus = str(torch.cuda.get_device_properties(0).pci_bus_id).lower()
            dom = int(getattr(torch.cuda.get_device_properties(0), "pci_domain_id", 0))
            slot = f"{dom:04x}:{bus:>02}" if len(bus) <= 2 else bus
        except Exception:
            slot = None
        drm = "/sys/class/drm"
        try:
            cards = sorted(c for c in os.listdir(drm) if c.startswith("card") and c[4:].isdigit())
        except OSError:
            cards = []
        for c in cards:
            dev = os.path.join(drm, c, "device")
            try:
                with open(os.path.join(dev, "uevent")) as fh:
                    ue = fh.read().lower()
            except OSError:
                continue
            if slot is None or (f"pci_slot_name={slot}" in ue or (":" + slot.split(":")[-1] + ":00.0") in ue):
                if os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
                    self.path = os.path.join(dev, "pp_dpm_sclk")
                    break

    def _read(self):
        with open(self.path) as fh:
            for line in fh:
                if "*" in line:
                    return float(line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", ""))
        return None

    def __enter__(self):
        import threading
        if self.path is None:
            return self

        def run():
            while not self._stop:
                try:
                    v = self._read()
                    if v:
                        self.samples.append(v)
                except (OSError, ValueError, IndexError):
                    return
                time.sleep(0.005)
        self._t = threading.Thread(target=run, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *a):
        self._stop = True
        if self.path is not None:
            self._t.join(timeout=1.0)

    def summary(self):
        if not self.samples:
            return None
        return {"sclk_mhz_median": float(np.median(self.samples)), "sclk_mhz_min": float(np.min(self.samples)),
                "sclk_mhz_max": float(np.max(self.samples)), "samples": len(self.samples)}


def cpu_baseline(w, inp, budget_s):
    """fp64 oracle, fwd+bwd, samples in order until the time budget is spent
    (shortest first for the sliding-window workload, whose samples are long)."""
    from oracle import attention as ora
    cores, host = host_info()
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    do, bias = inp.f64("dout"), inp.f64("bias")
    scale = 1.0 / np.sqrt(w.D) if w.scale is None else w.scale
    if w.mxfp8:
        # the MXFP8 oracle: the definition on the block-quantised values
        # (quantisation itself done before the timed samples)
        from oracle import mxfp8 as mx
        q, do = mx.quantize(q, inp.q_offsets)[2], mx.quantize(do, inp.q_offsets)[2]
        k, v = mx.quantize(k, inp.kv_offsets)[2], mx.quantize(v, inp.kv_offsets)[2]
    if w.qk_norm:
        return _cpu_baseline_qknorm(w, inp, q, k, v, do, scale, budget_s, cores)
    if w.rope:
        return _cpu_baseline_rope(w, inp, q, k, v, do, scale, budget_s, cores)
    # warm-up on a small sample
    lq, lk = inp.lq, inp.lk
    order = list(np.argsort(lq, kind="stable")) if w.window is not None else list(range(inp.B))
    ora.forward_sample(q, k, v, inp.q_offsets, inp.kv_offsets, int(order[0]), scale=scale, activation=w.act,
                       block_diagonal=w.block_diagonal, bias=bias, window=w.window)
    flops, n, done = 0.0, 0, []
    t_fwd = t_bwd = 0.0
    t0 = time.perf_counter()
    for b in order:
        b = int(b)
        ta = time.perf_counter()
        ora.forward_sample(q, k, v, inp.q_offsets, inp.kv_offsets, b, scale=scale, activation=w.act,
                           block_diagonal=w.block_diagonal, bias=bias, window=w.window)
        tb = time.perf_counter()
        ora.backward_sample(q, k, v, do, inp.q_offsets, inp.kv_offsets, b, scale=scale, activation=w.act,
                            block_diagonal=w.block_diagonal, bias=bias, want_dbias=w.want_dbias,
                            window=w.window)
        t_fwd += tb - ta
        t_bwd += time.perf_counter() - tb
        done.append(b)
        if w.block_diagonal:
            pairs = sum(min(64, int(lq[b]) - s) ** 2 for s in range(0, int(lq[b]), 64))
        elif w.window is not None:
            pairs = _window_pairs(int(lq[b]), w.window)
        else:
            pairs = int(lq[b]) * int(lk[b])
        flops += 3.5 * 4.0 * w.H * w.D * pairs
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    which = f"samples 0..{n - 1}" if w.window is None else \
        f"the {n} shortest samples (lengths {int(lq[done[0]])}..{int(lq[done[-1]])})"
    f_fwd = flops / 3.5
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{which} of {inp.B} (all {w.H} heads), fwd+bwd in float64, {dt:.1f} s",
            "fwd_s": round(t_fwd, 3), "bwd_s": round(t_bwd, 3),
            "fwd_tflops": f_fwd / max(t_fwd, 1e-9) / 1e12, "bwd_tflops": 2.5 * f_fwd / max(t_bwd, 1e-9) / 1e12,
            **host}


def _cpu_baseline_qknorm(w, inp, q, k, v, do, scale, budget_s, cores):
    """QK-norm, attention and both backwards per sample, in float64."""
    from oracle import attention as ora
    from oracle import qknorm as qn
    _, host = host_info()
    flops, n = 0.0, 0
    t0 = time.perf_counter()
    for b in range(inp.B):
        sq = slice(int(inp.q_offsets[b]), int(inp.q_offsets[b + 1]))
        sk = slice(int(inp.kv_offsets[b]), int(inp.kv_offsets[b + 1]))
        off_q, off_k = np.array([0, sq.stop - sq.start]), np.array([0, sk.stop - sk.start])
        qh, kh = qn.forward(q[sq])[0], qn.forward(k[sk])[0]
        ora.forward(qh, kh, v[sk], off_q, off_k, scale=scale, activation=w.act)
        dqh, dkh, _, _ = ora.backward(qh, kh, v[sk], do[sq], off_q, off_k, scale=scale, activation=w.act)
        qn.backward(q[sq], dqh)
        qn.backward(k[sk], dkh)
        flops += 3.5 * 4.0 * w.H * w.D * int(inp.lq[b]) * int(inp.lk[b])
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"samples 0..{n - 1} of {inp.B} (all {w.H} heads), QK-norm + attention, fwd+bwd in "
                      f"float64, {dt:.1f} s", **host}


def _cpu_baseline_rope(w, inp, q, k, v, do, scale, budget_s, cores):
    """RoPE, block attention and both backwards per sample, in float64."""
    from oracle import attention as ora
    from oracle import rope
    _, host = host_info()
    flops, n = 0.0, 0
    t0 = time.perf_counter()
    for b in range(inp.B):
        s_ = slice(int(inp.q_offsets[b]), int(inp.q_offsets[b + 1]))
        off = np.array([0, s_.stop - s_.start])
        qr, kr = rope.forward(q[s_], off), rope.forward(k[s_], off)
        ora.forward(qr, kr, v[s_], off, off, scale=scale, block_diagonal=True)
        dqr, dkr, _, _ = ora.backward(qr, kr, v[s_], do[s_], off, off, scale=scale, block_diagonal=True)
        rope.backward(dqr, off)
        rope.backward(dkr, off)
        L = int(inp.lq[b])
        flops += 3.5 * 4.0 * w.H * w.D * sum(min(64, L - s0) ** 2 for s0 in range(0, L, 64))
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"samples 0..{n - 1} of {inp.B} (all {w.H} heads), RoPE + block attention, fwd+bwd in "
                      f"float64, {dt:.1f} s", **host}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; multi-GPU runs (--gpus > 1) are not supported "
              "(attention has no cross-GPU exchange; the sharding design is per-sample data parallel)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calibration(args.copy_calib, args.steps)
        return
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.mfma_summary:
        mfma_summary(args)
        return

    import torch
    from jagged_variable_length_amd import attention as A
    from jagged_variable_length_amd import binding as Bd
    from jagged_variable_length_amd import inputs as gen

    cfg = args.config
    w = gen.WORKLOADS[cfg]
    inp = gen.make_inputs(cfg)  # the workload's canonical seed
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, w.H, w.D, act=w.act, block_diagonal=w.block_diagonal,
                           has_bias=w.bias, want_dbias=w.want_dbias,
                           in_dtype="mxfp8" if w.mxfp8 else w.dtype, out_dtype=w.out_dtype,
                           grad_dtype=w.grad_dtype, split_operands=w.split_operands, order=args.order,
                           num_workers=args.workers, dbias_dtype=w.dbias_dtype, window=w.window,
                           scale=w.scale, rope=w.rope)
    t0 = time.perf_counter()
    plan_ms = None
    op.upload()
    dev = {n: A.to_device(getattr(inp, n), w.dtype) for n in ("q", "k", "v", "dout")}
    bias = A.to_device(inp.bias, w.dtype) if inp.bias is not None else None
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    o = torch.empty(op.Tq, w.H, w.D, dtype=tdt[w.out_dtype], device="cuda")
    lse = torch.empty(op.Tq, w.H, dtype=torch.float32, device="cuda") if (w.act == "softmax" and not w.block_diagonal) else None
    dq = torch.empty(op.Tq, w.H, w.D, dtype=tdt[w.grad_dtype], device="cuda")
    dk = torch.empty(op.Tk, w.H, w.D, dtype=tdt[w.grad_dtype], device="cuda")
    dv = torch.empty_like(dk)
    dbias = torch.empty(int(op.info.bias_elems), dtype=tdt[w.dbias_dtype], device="cuda") if w.want_dbias else None
    # attention inputs and the gradients it produces for them: the normalised
    # copies of Q and K with QK-norm, else Q and K themselves
    q_in, k_in, dq_att, dk_att = dev["q"], dev["k"], dq, dk
    if w.qk_norm:
        q_in, k_in = torch.empty_like(dev["q"]), torch.empty_like(dev["k"])
        dq_att, dk_att = torch.empty_like(dq), torch.empty_like(dk)
        rq = torch.empty(op.Tq, w.H, dtype=torch.float32, device="cuda")
        rk = torch.empty(op.Tk, w.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    # plan creation cost (host only), measured on a fresh plan
    t1 = time.perf_counter()
    p2 = Bd.jattn_plan_create(op.desc, inp.q_offsets, inp.kv_offsets)
    plan_ms = (time.perf_counter() - t1) * 1e3
    Bd.jattn_plan_destroy(p2)

    if w.mxfp8:
        # the step starts from bf16 Q, K, V, dO: quantisation (the upstream
        # producer's job in the pages' design) is timed as part of it
        mq, mk, mv, mdo = op.mx_empty("q"), op.mx_empty("kv"), op.mx_empty("kv"), op.mx_empty("q")
        mx_sizes = (Bd.jattn_mx_sizes(op.plan, Bd.JATTN_MX_Q), Bd.jattn_mx_sizes(op.plan, Bd.JATTN_MX_KV))

        def quant():
            op.mx_quantize(dev["q"], "q", out=mq)
            op.mx_quantize(dev["k"], "kv", out=mk)
            op.mx_quantize(dev["v"], "kv", out=mv)
            op.mx_quantize(dev["dout"], "q", out=mdo)

        def mx_stage(s_):
            return lambda: op.mx_backward(mq, mk, mv, mdo, o=o, lse=lse, dq=dq, dk=dk, dv=dv, stages=s_)
        launches = [("quant", quant), ("fwd", lambda: op.mx_forward(mq, mk, mv, o=o, lse=lse))]
        if w.act == "softmax":
            launches.append(("prep", mx_stage(Bd.JATTN_BWD_PREP)))
        launches += [("dkdv", mx_stage(Bd.JATTN_BWD_DKDV)), ("dq", mx_stage(Bd.JATTN_BWD_DQ))]
    elif w.block_diagonal:
        launches = [("block_fwd", lambda: op.forward(dev["q"], dev["k"], dev["v"], o=o)),
                    ("block_bwd", lambda: op.backward(dev["q"], dev["k"], dev["v"], dev["dout"], dq=dq, dk=dk, dv=dv))]
    else:
        def fwd():
            op.forward(q_in, k_in, dev["v"], bias=bias, o=o, lse=lse)

        def stage(s):
            return lambda: op.backward(q_in, k_in, dev["v"], dev["dout"], o=o, lse=lse, bias=bias,
                                       dq=dq_att, dk=dk_att, dv=dv, dbias=dbias, stages=s)

        def qknorm():
            A.qk_norm(dev["q"], out=q_in, rnorm=rq)
            A.qk_norm(dev["k"], out=k_in, rnorm=rk)

        def qknorm_bwd():
            A.qk_norm_backward(dev["q"], dq_att, out=dq)
            A.qk_norm_backward(dev["k"], dk_att, out=dk)
        launches = [("qknorm", qknorm)] if w.qk_norm else []
        launches.append(("fwd", fwd))
        if rowstats_in_dq(w):
            # the order jattn_bwd runs: dQ (forming Di and LSE*log2e), then dK/dV
            launches += [("dq", stage(Bd.JATTN_BWD_DQ)), ("dkdv", stage(Bd.JATTN_BWD_DKDV))]
        else:
            if w.act == "softmax":
                launches.append(("prep", stage(Bd.JATTN_BWD_PREP)))
            launches += [("dkdv", stage(Bd.JATTN_BWD_DKDV)), ("dq", stage(Bd.JATTN_BWD_DQ))]
        if w.qk_norm:
            launches.append(("qknorm_bwd", qknorm_bwd))

    # Warm-up: the W steps asked for, then more (untimed) until the GPU has run
    # steps back to back for WARM_S seconds: after any pause the first steps run
    # slower (clock and caches ramping up), and the timed steps that follow
    # without a host pause should see the steady state.
    warm_steps, t_warm = 0, time.perf_counter()
    while warm_steps < args.warmup or time.perf_counter() - t_warm < WARM_S:
        for _ in range(4):
            for _, f in launches:
                f()
            warm_steps += 1
        torch.cuda.synchronize()

    ev = {n: [] for n, _ in launches}
    step_ev = []
    clock = ClockSampler(torch)
    with clock:
        t_start = time.perf_counter()
        for _ in range(args.steps):
            s0 = torch.cuda.Event(enable_timing=True)
            s0.record()
            for n, f in launches:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                f()
                b.record()
                ev[n].append((a, b))
            step_ev.append((s0, b))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
    times = {n: [a.elapsed_time(b) for a, b in lst] for n, lst in ev.items()}
    ms = {n: float(np.mean(t)) for n, t in times.items()}
    step_ms = [a.elapsed_time(b) for a, b in step_ev]

    F = float(op.info.flops_fwd)
    total_flops = 3.5 * F
    ms_per_step = wall * 1e3 / args.steps
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_F32_TFLOPS if w.dtype == "f32" else (PEAK_FP8_TFLOPS if w.mxfp8 else PEAK_BF16_TFLOPS)

    es = {"bf16": 2, "f32": 4}
    work = kernel_work(w, op.info, es[w.dtype], es[w.out_dtype], es[w.grad_dtype], es[w.dbias_dtype],
                       mx=mx_sizes if w.mxfp8 else None)
    dom = max(ms, key=lambda n: ms[n])
    nbytes, nflops = work[dom]
    t = ms[dom] * 1e-3
    ridge = peak / (PEAK_HBM_GBS / 1e3)
    if nflops / nbytes < ridge:
        achieved = nbytes / t / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = nflops / t / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak}
    roof["traffic"] = traffic_for(dom, cfg)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = nflops
    roof["ms_per_launch"] = ms[dom]

    kernels = {}
    for n in ms:
        b_, f_ = work[n]
        kernels[n] = {"ms": round(ms[n], 4), "ms_median": round(float(np.median(times[n])), 4),
                      "ms_min": round(float(np.min(times[n])), 4), "GB/s": round(b_ / (ms[n] * 1e-3) / 1e9, 1),
                      "TFLOP/s": round(f_ / (ms[n] * 1e-3) / 1e12, 2)}

    # MFMA counters of the dominant kernel, when profiles/mfma.json was taken
    # on these kernel sources: utilisation and the clock it ran at
    mf = mfma_for(dom, cfg)
    clock_info = None
    if mf:
        roof["mfma_util_pct"] = mf["mfma_util_pct"]
        clock_info = {"mhz": mf["clock_mhz"], "kernel": dom, "source": "GRBM_GUI_ACTIVE per XCD / dispatch duration "
                      "(rocprofv3 counters, profiles/mfma.json)"}
        # the dense MFMA peak at that clock: 1024 SIMDs x 1024 FLOP/clk (bf16), 2048 (fp8)
        per_clk = 2048 if w.mxfp8 else (256 if w.dtype == "f32" else 1024)
        roof["mfma_peak_at_clock_tflops"] = round(1024 * per_clk * mf["clock_mhz"] * 1e6 / 1e12, 1)
    clk = clock.summary()
    if clk:
        clock_info = dict(clock_info or {}, sysfs_sclk=clk)
    out = {
        "metric": "jagged attn fwd+bwd TFLOPs (valid tokens) and % of bf16 MFMA peak, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_events": {"median": round(float(np.median(step_ms)), 4), "min": round(float(np.min(step_ms)), 4),
                               "mean": round(float(np.mean(step_ms)), 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if w.mxfp8 else w.dtype,
        "data": "synthetic (seeded; lengths and value distributions of the workload)",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} D={w.D} {w.dtype} act={w.act}"
                               f"{' bias+dbias' if w.bias else ''}{' blockdiag64' if w.block_diagonal else ''}"
                               f"{f' window={w.window}' if w.window else ''}"
                               f"{f' qk-norm scale={w.scale}' if w.qk_norm else ''}"
                               f"{' rope' if w.rope else ''}{' mxfp8 (32x32 blocks, E4M3/E8M0)' if w.mxfp8 else ''}",
                   "workload_index": cfg, "Tq": op.Tq, "Tk": op.Tk,
                   "seed": cfg if w.seed is None else w.seed,
                   "flops_fwd": F, "flops_fwd_bwd": total_flops, "plan_ms_host": round(plan_ms, 3),
                   "order": args.order, "out_dtype": w.out_dtype, "grad_dtype": w.grad_dtype,
                   "dbias_dtype": w.dbias_dtype if w.want_dbias else None},
        "kernels": kernels,
        "roofline": roof,
        "clock": clock_info,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
