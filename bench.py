"""Bench: batched paged prefill attention on one MI355X.

One step = one call of the whole path (ppa_paged_prefill_attention through
the C ABI) over one synthetic batch already resident in HBM.  The default
workload is the chunked-context batch (8 requests, q_len U[128,1024] over a
U[0,512] cached prefix, 32 q / 8 kv heads, head_dim 128, page 32, HND
combined cache, seed 1002).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu]
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
sys.path.insert(0, ROOT)

METRIC = "prefill attention TFLOP/s (causal FLOPs), % bf16/fp8 MFMA peak; tokens/s"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 dense bf16 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2
PEAK_HBM_GBS = 8000.0

WORKLOAD_TEXT = {
    "tiny": "tiny: batch 2, q=kv=(37,64), 4 q / 2 kv heads, head_dim 64, page 16, HND split, seed 1001",
    "chunked": ("chunked context: batch 8, q_len U[128,1024] over prefix U[0,512], 32 q / 8 kv heads, "
                "head_dim 128, page 32, HND combined [pages,2,H,P,D], causal, seed 1002"),
    "llama3_8b": ("Llama-3-8B-shaped layer prefill: batch 16 x q=kv=2048, 32 q / 8 kv heads, head_dim 128, "
                  "page 64, HND split, causal, seed 1003"),
    "swa_sinks": ("sliding window 127 + sinks: batch 8, q_len U[512,4096] over prefix U[0,1024], 64 q / 8 kv "
                  "heads, head_dim 64, page 16, NHD split, seed 1004"),
    "fp8_long_prefix": ("long-prefix fp8 KV: batch 1, q 8192 over kv 32768, 64 q / 8 kv heads, head_dim 128, "
                        "page 64, HND split, e4m3fn K/V with per-tensor scales, seed 1005"),
    "decode": ("decode-shaped: batch 16, 1 new token over an 8191-token cached prefix, 32 q / 8 kv heads, "
               "head_dim 128, page 64, HND split, seed 1100 (HBM-bound; reported as K/V GB/s)"),
    "append_fp8": ("KV append: the 32768 new tokens of the Llama-3-8B-shaped batch (16 x 2048, 8 kv heads, "
                   "head_dim 128) quantised into an e4m3fn paged cache (page 64, HND split) at their slots"),
    "append_bf16": ("KV append: the 32768 new tokens of the Llama-3-8B-shaped batch (16 x 2048, 8 kv heads, "
                    "head_dim 128) copied into a bf16 paged cache (page 64, HND split) at their slots"),
}


def causal_pairs(case) -> int:
    """Number of (query row, key) pairs that pass the causal / window mask, per q head."""
    W = case["window_left"]
    total = 0
    for q, kv in zip(case["q_lens"], case["kv_lens"]):
        pre = kv - q
        pos = pre + np.arange(q, dtype=np.int64)
        n = pos + 1 if W < 0 else np.minimum(pos, W) + 1
        total += int(n.sum())
    return total


def algorithmic_bytes(case, out_elem_bytes: float = 2.0) -> int:
    """Compulsory HBM bytes: Q read + O written (``out_elem_bytes`` per
    element: 2 for bf16, 1/2 + 1/vec for MXFP4 codes and scales) + every KV
    token some query reaches, once."""
    D, Hq, Hkv = case["head_dim"], case["num_qo_heads"], case["num_kv_heads"]
    eb = 1 if case["kv_dtype"] != "bf16" else 2
    W = case["window_left"]
    tokens = sum(case["q_lens"])
    kv_reach = 0
    for q, kv in zip(case["q_lens"], case["kv_lens"]):
        if q == 0:
            continue
        lo = 0 if W < 0 else max(0, kv - q - W)
        kv_reach += kv - lo
    return int(tokens * Hq * D * (2 + out_elem_bytes)) + kv_reach * Hkv * D * eb * 2


def executed_flops(case, rows_per_workgroup: int = 256, kbk: int = 64, wave_rows: int = 32) -> float:
    """FLOPs of the MFMA work the kernel issues: every 32-row x 64-key
    wave-tile it does not skip (masked parts of diagonal and window tiles
    included), 4 * 32 * 64 * D each.  A count that follows the kernel's own
    tile-range and skip rules, for reporting executed beside causal FLOPs."""
    D, hq, hkv = case["head_dim"], case["num_qo_heads"], case["num_kv_heads"]
    G = hq // hkv
    gw = min(G, 16)
    n_hg = (G + gw - 1) // gw
    tq = rows_per_workgroup // gw
    W = case["window_left"]
    tiles = 0
    for q_len, kv_len in zip(case["q_lens"], case["kv_lens"]):
        prefix = kv_len - q_len
        for t0 in range(0, q_len, tq):
            ntok = min(tq, q_len - t0)
            for w in range(rows_per_workgroup // wave_rows):
                first = (w * wave_rows) // gw
                if first >= ntok:
                    continue
                last = min((w * wave_rows + wave_rows - 1) // gw, ntok - 1)
                khi = min(prefix + t0 + last, kv_len - 1)
                klo = max(prefix + t0 + first - W, 0) if W >= 0 else 0
                if khi >= klo:
                    tiles += khi // kbk - klo // kbk + 1
    return float(tiles) * hkv * n_hg * 4.0 * wave_rows * kbk * D


def device_info(torch, dev) -> dict:
    """What the device reports, to re-derive the roofline constants: compute
    units (torch's device properties), the highest shader clock in the
    driver's DPM table (sysfs, when readable), and the dense bf16 MFMA peak
    they imply at 4096 FLOP per CU per clock (the published 2516.6 TFLOP/s is
    256 CUs x 4096 x 2.4 GHz).  `peak` in the roofline stays the published
    figure."""
    import glob
    import re
    props = torch.cuda.get_device_properties(dev)
    cus = int(props.multi_processor_count)
    sclk = None
    for path in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            with open(path) as f:
                mhz = [int(m) for m in re.findall(r"(\d+)\s*[Mm][Hh]z", f.read())]
        except OSError:
            continue
        if mhz:
            sclk = max(sclk or 0, max(mhz))
    return {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": cus,
            "max_sclk_mhz": sclk,
            "bf16_peak_tflops_derived": None if sclk is None else round(cus * 4096 * sclk * 1e6 / 1e12, 1)}


def _sysfs_sclk_now():
    """The shader clock the driver reports as current: the starred line of
    pp_dpm_sclk (MHz), or None."""
    import glob
    import re
    for path in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        if m:
                            return int(m.group(1))
        except OSError:
            continue
    return None


_SMI = {"handle": None, "tried": False}


def _smi_gfxclk_now():
    """The graphics clock the power-management firmware reports now, averaged
    over the XCDs (amdsmi gpu_metrics current_gfxclks, MHz), or None.  Unlike
    the DPM level in pp_dpm_sclk (the clock the driver asks for), this follows
    the clock the part actually runs at under load."""
    if not _SMI["tried"]:
        _SMI["tried"] = True
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            _SMI["handle"] = handles[0] if handles else None
            _SMI["mod"] = amdsmi
        except Exception:
            _SMI["handle"] = None
    if _SMI["handle"] is None:
        return None
    try:
        m = _SMI["mod"].amdsmi_get_gpu_metrics_info(_SMI["handle"])
    except Exception:
        return None
    clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))]
    if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
        clks = [m["current_gfxclk"]]
    return float(np.mean(clks)) if clks else None


def sampled_clock(launch, seconds: float = 1.5):
    """The shader clock held under sustained load: the kernel is launched
    back to back for about `seconds` while a host thread samples the clock
    every 10 ms: the firmware's per-XCD graphics clock (amdsmi gpu_metrics)
    when it is readable, else the driver's current DPM level (sysfs
    pp_dpm_sclk, the starred line).  The firmware's figure refreshes with a
    lag, so samples from the first 40% of the window and idle readings
    (< 500 MHz) are dropped.  Returns {median, min, max, samples, source,
    dpm_level_median} or None when no readout is available."""
    import threading
    import torch
    samples = []
    dpm = []
    stop = threading.Event()
    use_smi = _smi_gfxclk_now() is not None

    def sample():
        while not stop.is_set():
            v = _smi_gfxclk_now() if use_smi else _sysfs_sclk_now()
            if v is not None:
                samples.append(v)
            d = _sysfs_sclk_now()
            if d is not None:
                dpm.append(d)
            time.sleep(0.010)

    th = threading.Thread(target=sample, daemon=True)
    t_end = time.perf_counter() + seconds
    th.start()
    while time.perf_counter() < t_end:
        for _ in range(20):
            launch()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    # the first samples can predate the ramp to load
    tail = [v for v in samples[(2 * len(samples)) // 5:] if v >= 500] or samples
    if not tail:
        return None
    dtail = dpm[len(dpm) // 4:] or dpm
    return {"median_mhz": round(float(np.median(tail)), 1), "min_mhz": round(float(min(tail)), 1),
            "max_mhz": round(float(max(tail)), 1), "samples": len(tail),
            "source": ("amdsmi gpu_metrics current_gfxclks (mean over the XCDs)" if use_smi
                       else "sysfs pp_dpm_sclk current level") + ", sampled every 10 ms under back-to-back launches",
            "dpm_level_median_mhz": float(np.median(dtail)) if dtail else None}


def time_config(config: str, steps: int, warmup: int, clock_seconds: float = 0.0) -> dict:
    """A second workload timed like the headline one (launches back to back,
    HIP events at the two ends of the region), for the extra keys of the
    bench line; with clock_seconds > 0, also the clock it holds (sampled_clock)
    and its fraction of the peak at that clock."""
    import torch

    import paged_kv_prefill_varlen_amd as ppa
    from workloads import make_case

    dev = torch.device("cuda:0")
    case = make_case(config)
    q = case["query"].to(dev)
    kv = case["kv_cache"]
    kv = tuple(t.to(dev) for t in kv) if isinstance(kv, tuple) else kv.to(dev)
    out = torch.empty_like(q)
    ws = torch.zeros(ppa.WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    p = ppa.make_params(q, kv, ws, case["block_tables"].to(dev), case["seq_lens"].to(dev), case["max_q_len"],
                        case["max_kv_len"], case["bmm1_scale"], case["bmm2_scale"], case["batch_size"],
                        case["cum_seq_lens_q"].to(dev), case["cum_seq_lens_kv"].to(dev), case["window_left"], out,
                        case["kv_layout"], None if case["sinks"] is None else case["sinks"].to(dev))
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        ppa.ppa_paged_prefill_attention(p, stream.cuda_stream)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        ppa.ppa_paged_prefill_attention(p, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    flops = 4.0 * case["head_dim"] * case["num_qo_heads"] * causal_pairs(case)
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": WORKLOAD_TEXT[config], "kernel_ms": round(ms, 5), "causal_gflop": round(flops / 1e9, 3),
           "tflops": round(tf, 3), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
           "tokens_per_s": round(sum(case["q_lens"]) / (ms * 1e-3), 1), "steps": steps}
    if clock_seconds > 0:
        clock = sampled_clock(lambda: ppa.ppa_paged_prefill_attention(p, stream.cuda_stream), clock_seconds)
        res["clock"] = clock
        if clock is not None:
            res["frac_at_measured_clock"] = round(tf / (PEAK_BF16_TFLOPS * clock["median_mhz"] / 2400.0), 4)
    return res


def cpu_baseline(case, budget_s: float = 12.0):
    """Time the CPU oracle (as it stands) on whole passes over the same batch,
    repeated until about budget_s of work; report causal TFLOP/s."""
    from threadpoolctl import threadpool_info

    from oracle.case_io import oracle_inputs
    from oracle.paged_attention import paged_prefill_attention

    a = oracle_inputs(case)
    t_total = 0.0
    passes = 0
    while t_total < budget_s or passes == 0:
        t = time.perf_counter()
        paged_prefill_attention(**a)
        t_total += time.perf_counter() - t
        passes += 1
    flops = passes * 4.0 * case["head_dim"] * case["num_qo_heads"] * causal_pairs(case)
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(flops / t_total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "host_cores": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle, {passes} full pass(es) over the same batch "
                   f"({sum(case['q_lens'])} query tokens each), {t_total:.1f} s"),
    }


def _elf_sections(b: bytes, names) -> dict:
    """Named sections of a little-endian ELF64 image."""
    import struct
    shoff, = struct.unpack_from("<Q", b, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)

    def header(i):
        return struct.unpack_from("<IIQQQQ", b, shoff + i * shentsize)

    strtab = header(shstrndx)[4]
    out = {}
    for i in range(shnum):
        name, _, _, _, off, size = header(i)
        n = b[strtab + name: b.index(b"\0", strtab + name)].decode()
        if n in names:
            out[n] = b[off: off + size]
    return out


def kernel_code_digest(lib_path: str, kernel: str) -> str:
    """sha256 over the gfx950 machine code and kernel descriptor of one
    kernel of the library (the function symbol containing `kernel` and its
    `.kd` descriptor, found through the code object's symbol table): ties
    stored counter readings to the kernel they were taken on.  Host-only
    changes and changes to other kernels keep it."""
    import hashlib
    import struct
    with open(lib_path, "rb") as f:
        b = f.read()
    bundle = _elf_sections(b, {".hip_fatbin"}).get(".hip_fatbin", b"")
    if bundle[:24] != b"__CLANG_OFFLOAD_BUNDLE__":
        return ""
    n, = struct.unpack_from("<Q", bundle, 24)
    pos = 32
    for _ in range(n):
        off, size, tlen = struct.unpack_from("<QQQ", bundle, pos)
        triple = bundle[pos + 24: pos + 24 + tlen].decode()
        pos += 24 + tlen
        if not triple.endswith("gfx950"):
            continue
        obj = bundle[off: off + size]
        shoff, = struct.unpack_from("<Q", obj, 0x28)
        shentsize, shnum, shstrndx = struct.unpack_from("<HHH", obj, 0x3A)
        hdrs = [struct.unpack_from("<IIQQQQIIQQ", obj, shoff + i * shentsize) for i in range(shnum)]
        names = [obj[hdrs[shstrndx][4] + h[0]: obj.index(b"\0", hdrs[shstrndx][4] + h[0])].decode() for h in hdrs]
        symtab = hdrs[names.index(".symtab")]
        strtab = hdrs[symtab[6]]   # sh_link
        h = hashlib.sha256()
        found = 0
        for i in range(symtab[5] // 24):
            st_name, _, _, shndx, value, sz = struct.unpack_from("<IBBHQQ", obj, symtab[4] + 24 * i)
            name = obj[strtab[4] + st_name: obj.index(b"\0", strtab[4] + st_name)].decode()
            if kernel not in name or shndx == 0 or shndx >= len(hdrs) or sz == 0:
                continue
            sec = hdrs[shndx]   # symbol value is an address inside this section
            start = sec[4] + value - sec[3]
            h.update(name.encode())
            h.update(obj[start: start + sz])
            found += 1
        return h.hexdigest() if found else ""
    return ""


# the kernel the stored counters of a bf16 workload were taken on
def _kernel_symbol(case) -> str:
    fp8 = case["kv_dtype"] != "bf16"
    return "paged_prefill_persistentILi%dELb%dELb1ELb%dE" % (case["head_dim"], 1 if fp8 else 0,
                                                             1 if fp8 and case["head_dim"] == 128 else 0)


def _library_path() -> str:
    import paged_kv_prefill_varlen_amd as ppa
    return ppa.library_path()


def stored_traffic(config: str):
    """HBM bytes per launch from the committed counter summary for this
    workload, or None when it is missing or was taken on other kernels."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_code_sha256") != kernel_code_digest(_library_path(), d.get("kernel_symbol", "?")):
        return None
    return d.get("traffic_bytes")


def copy_calibration(nbytes: int = 1 << 28, reps: int = 3) -> None:
    """A plain streaming kernel of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters: each add dispatch reads nbytes and writes nbytes."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def traffic_summary(config: str, dirs) -> None:
    """Write profiles/hbm_traffic_<config>.json from four rocprofv3 --pmc
    output folders (csv): FETCH_SIZE and WRITE_SIZE of the workload's
    attention kernel, then of the copy calibration.  The counters read KiB
    per dispatch; each is scaled by the bytes the calibration's add kernel is
    known to move (256 MiB each way) over what the same counter read for it."""
    import csv
    import statistics

    def values(folder, counter, match, last=None):
        with open(os.path.join(folder, "run_counter_collection.csv")) as f:
            v = [float(r["Counter_Value"]) for r in csv.DictReader(f)
                 if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
        return v[-last:] if last else v

    from workloads import make_case
    sym = _kernel_symbol(make_case(config))
    kern = lambda n: "paged_prefill" in n          # noqa: E731
    add = lambda n: "elementwise" in n             # noqa: E731
    fetch = values(dirs[0], "FETCH_SIZE", kern)
    write = values(dirs[1], "WRITE_SIZE", kern)
    cfetch = values(dirs[2], "FETCH_SIZE", add, 3)
    cwrite = values(dirs[3], "WRITE_SIZE", add, 3)
    kib = (1 << 28) / 1024
    fs = kib / statistics.mean(cfetch)
    ws = kib / statistics.mean(cwrite)
    rd = statistics.mean(fetch) * 1024 * fs
    wr = statistics.mean(write) * 1024 * ws
    out = {
        "kernel": "paged_prefill_persistent (the workload's bf16 or fp8 instance)",
        "workload": config,
        "fetch_kib_per_dispatch": [round(x, 1) for x in fetch],
        "write_kib_per_dispatch": [round(x, 1) for x in write],
        "calibration": {"kernel": "torch.add(src, 1.0, out=dst), float32, 256 MiB each way",
                        "fetch_kib": [round(x, 1) for x in cfetch], "write_kib": [round(x, 1) for x in cwrite],
                        "fetch_scale": round(fs, 5), "write_scale": round(ws, 5)},
        "read_bytes": int(rd),
        "write_bytes": int(wr),
        "traffic_bytes": int(rd + wr),
        "kernel_symbol": sym,
        "kernel_code_sha256": kernel_code_digest(_library_path(), sym),
        "commands": [
            "cd /tmp && export TMPDIR=/tmp",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch dir> -o run -- python3 bench.py "
            f"--steps 2 --warmup 1 --no-cpu --cold-iters 0 --config {config}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write dir> -o run -- python3 bench.py "
            f"--steps 2 --warmup 1 --no-cpu --cold-iters 0 --config {config}",
            "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <copy dirs> -o run -- "
            "python3 bench.py --copy-calibration",
            f"python3 bench.py --config {config} --traffic-summary <fetch dir> <write dir> <copy fetch dir> "
            "<copy write dir>",
        ],
    }
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{config}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({"wrote": path, "traffic_bytes": out["traffic_bytes"]}))


def bench_append(args) -> None:
    """Time ppa_append_paged_kv (HBM-bound): new K/V read, cache written."""
    import torch

    import paged_kv_prefill_varlen_amd as ppa
    from workloads import make_case

    fp8 = args.config == "append_fp8"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = make_case("llama3_8b", kv_dtype="fp8_e4m3fn" if fp8 else "bf16")
    P = case["page_size"]
    bt = case["block_tables"].numpy()
    slots = []
    for b, (q, kv) in enumerate(zip(case["q_lens"], case["kv_lens"])):
        pos = np.arange(kv - q, kv)
        slots.append(bt[b, pos // P].astype(np.int64) * P + pos % P)
    slots = torch.from_numpy(np.concatenate(slots)).to(dev)
    n = slots.numel()
    H, D = case["num_kv_heads"], case["head_dim"]
    g = torch.Generator(device=dev).manual_seed(5)
    k_new = torch.randn((n, H, D), generator=g, device=dev).to(torch.bfloat16)
    v_new = torch.randn((n, H, D), generator=g, device=dev).to(torch.bfloat16)
    kv = tuple(t.to(dev) for t in case["kv_cache"])
    q_stub = torch.empty((1, 1, D), dtype=torch.bfloat16, device=dev)
    i32 = torch.zeros(2, dtype=torch.int32, device=dev)
    cache = ppa.make_params(q_stub, kv, None, torch.zeros((1, 1), dtype=torch.int32, device=dev), i32[:1], 0, 0,
                            1.0, 1.0, 0, i32, None, -1, q_stub, "HND")
    a = ppa.make_append_params(k_new, v_new, slots, 0.02, 0.03)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        ppa.ppa_append_paged_kv(cache, a, stream.cuda_stream)
    torch.cuda.synchronize(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        ppa.ppa_append_paged_kv(cache, a, stream.cuda_stream)
    t1.record(stream)
    torch.cuda.synchronize(dev)
    ms_per_step = t0.elapsed_time(t1) / args.steps
    launch_ms = ms_per_step
    eb = 1 if fp8 else 2
    alg = n * H * D * 2 * 2 + n * H * D * eb * 2 + n * 8   # read new K/V, write cache, slots
    gbs = alg / (ms_per_step * 1e-3) / 1e9
    kgbs = alg / (launch_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "KV append GB/s (new K/V read + cache written)", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config], "name": args.config, "tokens": n,
                   "parallelism": "none (one GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(kgbs / PEAK_HBM_GBS, 4), "traffic": None, "algorithmic_bytes": alg,
                     "kernel_ms": round(launch_ms, 5), "kernel": "append_kernel<%s>" % ("fp8" if fp8 else "bf16")},
        "cpu_baseline": None,
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="chunked", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--fp8-compute", choices=["auto", "0", "1"], default="auto",
                    help="fp8 cache: 1 runs both products on the fp8 MFMA (Q and P rounded to e4m3fn), 0 "
                         "widens the codes to bf16; auto: 1 at head_dim 128")
    ap.add_argument("--kv-splits", default="auto",
                    help="split-KV chunks per work item (0: none; auto: the library's planner, the default)")
    ap.add_argument("--cold-iters", type=int, default=10,
                    help="extra launches, each after writing a 512 MB buffer (cold caches); 0 to skip")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "mxfp4"],
                    help="output: bf16, or MXFP4 codes + E8M0 block scales")
    ap.add_argument("--o-sf-vec-size", type=int, default=32, choices=[16, 32])
    ap.add_argument("--clock-seconds", type=float, default=2.0,
                    help="seconds of back-to-back launches while sampling the shader clock (0: skip)")
    ap.add_argument("--no-llama3", dest="also_llama3", action="store_false",
                    help="chunked workload: skip timing the Llama-3-8B-shaped batch as well")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=4, metavar="DIR",
                    help="write profiles/hbm_traffic_<config>.json from rocprofv3 FETCH_SIZE / WRITE_SIZE "
                         "folders of the workload and of --copy-calibration")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.config, args.traffic_summary)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the kernel shards by kv head or request with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    if args.config.startswith("append"):
        bench_append(args)
        return

    import torch

    import paged_kv_prefill_varlen_amd as ppa
    from workloads import make_case

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = make_case(args.config)
    q = case["query"].to(dev)
    kv = case["kv_cache"]
    kv = tuple(t.to(dev) for t in kv) if isinstance(kv, tuple) else kv.to(dev)
    bt = case["block_tables"].to(dev)
    sl = case["seq_lens"].to(dev)
    cuq = case["cum_seq_lens_q"].to(dev)
    cukv = case["cum_seq_lens_kv"].to(dev)
    sinks = None if case["sinks"] is None else case["sinks"].to(dev)
    if args.out_dtype == "mxfp4":
        out = ppa.empty_mxfp4(q.shape[0], q.shape[1], q.shape[2], dev, args.o_sf_vec_size, 1.0)
    else:
        out = torch.empty_like(q)
    # zeroed scheduler workspace: persistent workgroups pull balanced work
    # (larger with split-KV: it also holds the partial states)
    # "auto": the library's planner picks the split count for this shape and
    # device, within a workspace sized for up to 256 splits (at most 256 MiB)
    auto = args.kv_splits == "auto"
    splits = 256 if auto else int(args.kv_splits)
    f8c = case["kv_dtype"] != "bf16" and (args.fp8_compute == "1" or
                                          (args.fp8_compute == "auto" and case["head_dim"] == 128))
    p = ppa.make_params(q, kv, None, bt, sl, case["max_q_len"], case["max_kv_len"], case["bmm1_scale"],
                        case["bmm2_scale"], case["batch_size"], cuq, cukv, case["window_left"], out,
                        case["kv_layout"], sinks, kv_splits=splits, fp8_compute=f8c)
    ws_bytes = ppa.ppa_workspace_bytes(p)
    if auto:
        ws_bytes = max(ppa.WORKSPACE_BYTES, min(ws_bytes, 256 << 20))
    workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    p = ppa.make_params(q, kv, workspace, bt, sl, case["max_q_len"], case["max_kv_len"], case["bmm1_scale"],
                        case["bmm2_scale"], case["batch_size"], cuq, cukv, case["window_left"], out,
                        case["kv_layout"], sinks, kv_splits=0 if auto else splits, fp8_compute=f8c)
    if auto:
        p.kv_splits = ppa.ppa_plan_kv_splits(p)
    args.kv_splits = int(p.kv_splits)
    st, msg = ppa.ppa_validate_metadata_host(p, case["cum_seq_lens_q"], case["cum_seq_lens_kv"],
                                             case["seq_lens"], case["block_tables"])
    if st != 0:
        raise SystemExit(f"workload metadata invalid: {msg}")
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream

    for _ in range(args.warmup):
        ppa.ppa_paged_prefill_attention(p, handle)
    torch.cuda.synchronize(dev)

    # the timed region: K launches back to back on the launch stream, HIP
    # events only at its two ends, so the average launch duration is the
    # region over K (nothing recorded between launches)
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t_begin.record(stream)
    for _ in range(args.steps):
        ppa.ppa_paged_prefill_attention(p, handle)
    t_end.record(stream)
    torch.cuda.synchronize(dev)
    total_ms = t_begin.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    launch_ms = ms_per_step
    # a second pass with each launch bracketed by its own events: their
    # median (which adds the dispatch latency to each launch)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        ppa.ppa_paged_prefill_attention(p, handle)
        ends[i].record(stream)
    torch.cuda.synchronize(dev)
    launch_times = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    # cold cache: a 512 MB buffer is written between launches (evicting L2
    # and the Infinity Cache); only the launch itself is timed
    cold_ms = None
    if args.cold_iters > 0:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = []
        for i in range(args.cold_iters):
            scratch.fill_(i & 0xFF)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ppa.ppa_paged_prefill_attention(p, handle)
            e1.record(stream)
            torch.cuda.synchronize(dev)
            cold.append(e0.elapsed_time(e1))
        cold_ms = float(np.median(cold))
        del scratch

    # the shader clock held under sustained launches of the same call
    clock = None
    if args.clock_seconds > 0:
        clock = sampled_clock(lambda: ppa.ppa_paged_prefill_attention(p, handle), args.clock_seconds)

    flops = 4.0 * case["head_dim"] * case["num_qo_heads"] * causal_pairs(case)
    tokens = sum(case["q_lens"])
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    kernel_tflops = flops / (launch_ms * 1e-3) / 1e12
    fp8 = case["kv_dtype"] != "bf16"
    # an fp8 cache at head_dim 128 runs both products on the fp8 MFMA (Q and
    # P rounded to e4m3fn): the contraction's own peak is the fp8 one
    mma_fp8 = bool(p.fp8_compute)
    peak = PEAK_FP8_TFLOPS if mma_fp8 else PEAK_BF16_TFLOPS
    alg_bytes = algorithmic_bytes(case, 2.0 if args.out_dtype == "bf16" else 0.5 + 1.0 / args.o_sf_vec_size)
    # the bound follows the arithmetic intensity: below the ridge
    # (peak FLOP/s over HBM bytes/s) the compulsory bytes bound the kernel
    ai = flops / alg_bytes
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    hbm = args.config == "decode" or ai < ridge
    attainable = min(peak, ai * PEAK_HBM_GBS / 1e3)
    if hbm:   # the compulsory bytes bound it: report bandwidth against HBM
        kernel_gbs = alg_bytes / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(kernel_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(kernel_gbs / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(kernel_tflops, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(kernel_tflops / peak, 4),
                "traffic": stored_traffic(args.config) if args.out_dtype == "bf16" else None}
    roof.update({"algorithmic_bytes": alg_bytes, "kernel_ms": round(launch_ms, 5),
                 "bracketed_launch_ms_median": round(float(np.median(launch_times)), 5),
                 "cold_kernel_ms_median": None if cold_ms is None else round(cold_ms, 5),
                 "flop_per_byte": round(ai, 1),
                 "attainable_tflops": round(attainable, 1),
                 "frac_attainable": round(kernel_tflops / attainable, 4),
                 "executed_tflops": round(executed_flops(case) / (launch_ms * 1e-3) / 1e12, 3),
                 "kernel": "paged_prefill_persistent<%d,%s>%s" % (case["head_dim"],
                                                                  ("fp8 MFMA" if mma_fp8 else "fp8 widened to bf16")
                                                                  if fp8 else "bf16",
                                                                  " + merge" if args.kv_splits > 1 else "")})
    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if mma_fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config], "name": args.config,
                   "query_tokens": tokens, "causal_gflop": round(flops / 1e9, 3),
                   "kv_splits": args.kv_splits, "kv_splits_from": "planner" if auto else "argument", "out": args.out_dtype if args.out_dtype == "bf16"
                   else f"mxfp4/{args.o_sf_vec_size}", "parallelism": "none (one GPU)"},
        "tokens_per_s": round(tokens / (ms_per_step * 1e-3), 1),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "pct_fp8_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2) if mma_fp8 else None,
        "roofline": roof,
        "cpu_baseline": None,
        "device": device_info(torch, dev),
    }
    # peak and fraction at the clock the part held, beside the spec clock
    # (2.4 GHz) that `peak` uses
    if clock is not None and roof["bound"] == "mfma":
        peak_measured = peak * clock["median_mhz"] / 2400.0
        roof["measured_sclk_mhz"] = clock["median_mhz"]
        roof["peak_at_measured_clock"] = round(peak_measured, 1)
        roof["frac_at_measured_clock"] = round(kernel_tflops / peak_measured, 4)
    line["clock"] = clock
    # the other reading of the gate's "config 2": the Llama-3-8B-shaped batch
    if args.config == "chunked" and args.also_llama3:
        # (its own clock: it draws more power than the headline batch)
        line["llama3_8b"] = time_config("llama3_8b", max(5, args.steps // 2), 3, args.clock_seconds)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
