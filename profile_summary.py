"""Profile the benchmark's workloads with rocprofv3 and write the summaries in profiles/.

Two steps, because the GPU run and the summary may happen on different machines:

  python3 profile_summary.py run NAME [--out DIR]
      On a machine with the GPU: runs bench.py under rocprofv3 as child processes, one
      pass each -- the kernel trace with statistics, then FETCH_SIZE, then WRITE_SIZE, then
      the named profile's extra counter sets -- writing raw CSV under DIR/NAME (default
      rocprof_out).  Each pass runs under its own time limit; the first failure stops
      the sequence.  This script itself never touches the GPU.

  python3 profile_summary.py summarize NAME [--out DIR]
      Reads DIR/NAME and writes profiles/NAME.txt: every command, the per-kernel durations
      (all dispatches, and the timed dispatches at the end of the run), the calibrated HBM
      traffic per dispatch against the kernel's algorithmic bytes, and the extra counters
      with the ratios derived from them.  The traffic of each measured kernel goes to
      profiles/traffic.json together with a hash of the kernel sources it was measured on;
      bench.py reports it only while those sources are unchanged.

Calibration: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) count requests between the L2
and the memory fabric.  The `hbm_copy` profile times a plain 1 GiB copy (1 GiB read, 1
GiB written); the ratio of those known bytes to the counters scales every other kernel's
counters.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "microscaled_fp4_quantization_block_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC = os.path.join(PROFILES, "traffic.json")

SQ_PASS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
           "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]

M_, N_, K_ = 8192, 28672, 8192
DEVICE_HPP = ["fp4_device.hpp"]

#: name -> what to run and which kernels to report.  `kernels`: substring of the kernel
#: name -> (traffic.json key or None, sources, algorithmic bytes per dispatch or None,
#: FLOP per dispatch or None).
CASES = {
    "hbm_copy": dict(
        title="plain 1 GiB device-to-device copy (counter calibration)",
        bench=["--workload", "hbm_copy"], steps=20, timed=20, pmc=[],
        kernels={"copyBuffer": (None, [], 2 << 30, None)}),
    "w4a4_8192x28672x8192": dict(
        title="W4A4 step: k_quant_mx<bf16,H32> on one of eight rotating A batches (bf16 8192x8192), then "
              "k_gemm MXFP4 8192x28672x8192, bf16 out (one extra k_quant_mx dispatch quantizes the 28672x8192 "
              "weights, and the settle phase repeats the step for a second before the timed steps)",
        bench=["--workload", "w4a4_gemm"], steps=20, timed=20, pmc=[SQ_PASS],
        kernels={"k_gemm": ("gemm_w4a4", ["gemm.hip", "gemm_core.hpp"] + DEVICE_HPP, 630194176, 2.0 * M_ * N_ * K_),
                 "k_quant_mx": ("quant_mx_h32_a", ["quant.hip"] + DEVICE_HPP, 169869312, None)}),
    "w4a4_shard_8192x3584x8192": dict(
        title="W4A4 step at one GPU's column shard of eight: k_quant_mx<bf16,H32> on one of eight rotating A "
              "batches (bf16 8192x8192), then k_gemm MXFP4 8192x3584x8192 (the first 3584 of the 28672 weight "
              "rows), bf16 out",
        bench=["--workload", "w4a4_shard"], steps=20, timed=20, pmc=[SQ_PASS],
        kernels={"k_gemm": ("gemm_w4a4_shard", ["gemm.hip", "gemm_core.hpp"] + DEVICE_HPP, 109969408,
                            2.0 * M_ * 3584 * K_),
                 "k_quant_mx": (None, [], 169869312, None)}),
    "k_quant_mx_h32_4096x4096": dict(
        title="Hadamard-32 MXFP4 quantization, bf16 4096x4096 with 41 outlier channels x50 (rotating buffers)",
        bench=["--workload", "mxfp4_h32", "--op", "quant"], steps=100, timed=100, pmc=[SQ_PASS],
        kernels={"k_quant_mx": ("mxfp4_h32_quant", ["quant.hip"] + DEVICE_HPP, 42467328, None)}),
    "k_dequant_mx_h32_bf16_4096x4096": dict(
        title="MXFP4 dequantization with inverse Hadamard-32 to bf16, 4096x4096 (rotating buffers)",
        bench=["--workload", "mxfp4_h32", "--op", "dequant"], steps=100, timed=100, pmc=[SQ_PASS],
        kernels={"k_dequant": ("mxfp4_h32_dequant", ["quant.hip"] + DEVICE_HPP, 42467328, None)}),
    "k_quant_nv_h16_4096x4096": dict(
        title="Hadamard-16 NVFP4 quantization with a calibrated (static) tensor scale, bf16 4096x4096 with 41 "
              "outlier channels x50 (rotating buffers)",
        bench=["--workload", "nvfp4_h16", "--op", "quant"], steps=100, timed=100, pmc=[SQ_PASS],
        kernels={"k_quant_nv": ("nvfp4_h16_quant", ["quant.hip"] + DEVICE_HPP, 42991620, None)}),
    "k_dequant_nv_h16_bf16_4096x4096": dict(
        title="NVFP4 dequantization with inverse Hadamard-16 to bf16, 4096x4096 (rotating buffers)",
        bench=["--workload", "nvfp4_h16", "--op", "dequant"], steps=100, timed=100, pmc=[SQ_PASS],
        kernels={"k_dequant": ("nvfp4_h16_dequant", ["quant.hip"] + DEVICE_HPP, 42991620, None)}),
    "k_pack_8192x8192": dict(
        title="dual-scale FP4 pack with the two-level FWHT, bf16 8192x8192 Student-t(4) (rotating buffers)",
        bench=["--workload", "dualscale_pack", "--op", "quant"], steps=50, timed=50, pmc=[SQ_PASS],
        kernels={"k_pack": ("dualscale_pack_quant", ["pack.hip"] + DEVICE_HPP, 174063616, None)}),
    "k_unpack_8192x8192": dict(
        title="dual-scale FP4 unpack with the two-level FWHT to bf16, 8192x8192 (rotating buffers)",
        bench=["--workload", "dualscale_pack", "--op", "dequant"], steps=50, timed=50, pmc=[SQ_PASS],
        kernels={"k_unpack": ("dualscale_pack_dequant", ["pack.hip"] + DEVICE_HPP, 174063616, None)}),
    "k_arcquant_4096x4096_S256": dict(
        title="ARCQuant fused RMSNorm + reorder + NVFP4 primary + residual (S = 256), bf16 4096x4096, "
              "static tensor scale (rotating buffers)",
        bench=["--workload", "arcquant"], steps=100, timed=100, pmc=[SQ_PASS],
        kernels={"k_arcquant": ("arcquant_quant", ["arcquant.hip"] + DEVICE_HPP, 43597828, None)}),
    "k_arcquant_gamma_4096x4096_S256": dict(
        title="ARCQuant NVFP4 with a gain vector (gamma uniform in [0.5, 1.5]), S = 256, bf16 4096x4096, "
              "static tensor scale (rotating buffers)",
        bench=["--workload", "arcquant_gamma"], steps=100, timed=100, pmc=[SQ_PASS],
        kernels={"k_arcquant": ("arcquant_gamma_quant", ["arcquant.hip"] + DEVICE_HPP, 43614212, None)}),
    "k_arcquant_mx_4096x4096_S256": dict(
        title="ARCQuant MXFP4 flavour (E8M0 per 32), S = 256, bf16 4096x4096 (rotating buffers)",
        bench=["--workload", "arcquant_mx"], steps=100, timed=100, pmc=[SQ_PASS],
        kernels={"k_arcquant": ("arcquant_mx_quant", ["arcquant.hip"] + DEVICE_HPP, 43040768, None)}),
    "nvfp4_roundtrip_256x1024": dict(
        title="NVFP4 quantize + dequantize round trip, fp32 256x1024, dynamic tensor scale",
        bench=["--workload", "nvfp4_roundtrip"], steps=100, timed=100, pmc=[],
        kernels={"k_quant_nv": (None, ["quant.hip"] + DEVICE_HPP, 1196036, None),
                 "k_dequant": (None, ["quant.hip"] + DEVICE_HPP, 1196036, None),
                 "k_amax": (None, [], None, None)}),
    "arcquant_gemm_4096x14336x4352": dict(
        title="ARCQuant augmented GEMM step: k_arcquant<MXFP4> (S = 256) then k_gemm 4096x14336x4352, against "
              "the same step at S = 0 (k_gemm 4096x14336x4096)",
        bench=["--workload", "arcquant_gemm"], steps=20, timed=None, pmc=[],
        kernels={"k_gemm": (None, [], None, None), "k_arcquant": (None, [], None, None)}),
    "w4a4_fused_8192x28672x8192": dict(
        title="fused-quantization experiment: k_gemm<8, true> (each tile rotates and quantizes its bf16 A "
              "rows into LDS) against the two-launch step k_quant_mx<bf16,H32> + k_gemm<8, false>, W4A4 "
              "8192x28672x8192",
        bench=["--workload", "w4a4_fused"], steps=5, timed=None, pmc=[],
        kernels={"k_gemm<8, true>": (None, [], None, 2.0 * M_ * N_ * K_),
                 "k_gemm<8, false>": (None, [], None, 2.0 * M_ * N_ * K_),
                 "k_quant_mx": (None, [], None, None)}),
    "hbm_read_1GiB": dict(
        title="roofline probe: read-only HBM stream, 1 GiB per launch", bench=["--workload", "hbm_read"],
        steps=20, timed=20, pmc=[], kernels={"k_hbm_read": (None, [], 1 << 30, None)}),
    "hbm_read_32MiB": dict(
        title="roofline probe: read-only HBM stream, 32 MiB per launch (the bf16 4096x4096 working set), "
              "rotating buffers", bench=["--workload", "hbm_read", "--bytes", str(32 << 20)],
        steps=200, timed=200, pmc=[], kernels={"k_hbm_read": (None, [], 32 << 20, None)}),
    "mfma_peak": dict(
        title="roofline probe: register-only FP4 MFMA loop, operand bytes changed every iteration",
        bench=["--workload", "mfma_peak", "--mode", "2"], steps=10, timed=10, pmc=[SQ_PASS],
        kernels={"k_mfma_loop": (None, [], None, 1024.0 * 8 * 20000 * 8 * 131072)}),
    "mfma_peak_constant": dict(
        title="roofline probe: register-only FP4 MFMA loop, constant operand bytes",
        bench=["--workload", "mfma_peak", "--mode", "0"], steps=10, timed=10, pmc=[],
        kernels={"k_mfma_loop": (None, [], None, 1024.0 * 8 * 20000 * 8 * 131072)}),
}


def code_text(src):
    """C/C++ source without its comments and with every run of white space collapsed to one
    space: the text that decides the compiled kernel.  String and character literals are
    kept as written."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == "/" and src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif c == "/" and src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_sha(files):
    """SHA-256 (first 16 hex digits) of the listed kernel sources' code text (comments and
    layout do not count), in order."""
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _commands(name, out):
    c = CASES[name]
    base = [sys.executable, os.path.join(ROOT, "bench.py"), *c["bench"], "--no-cpu"]
    d = os.path.join(out, name)
    cmds = [("trace", 300, ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                            os.path.join(d, "trace"), "-o", "run", "--", *base, "--steps", str(c["steps"]),
                            "--warmup", "2"])]
    passes = [["FETCH_SIZE"], ["WRITE_SIZE"]] + c["pmc"]
    for i, counters in enumerate(passes):
        tag = counters[0] if i < 2 else f"pmc{i - 1}"
        cmds.append((tag, 120, ["rocprofv3", "--pmc", *counters, "--output-format", "csv", "-d",
                                os.path.join(d, tag), "-o", "run", "--", *base, "--steps", "3", "--warmup", "1",
                                "--settle", "0"]))
    return cmds


def _display(cmd):
    out = []
    for a in cmd:
        if a == sys.executable:
            a = "python3"
        a = a.replace(ROOT + os.sep, "")
        out.append(a)
    return " ".join(out)


def run(name, out):
    out = os.path.abspath(out)     # the profiler runs from /tmp: a relative path would land there
    env = dict(os.environ, TMPDIR="/tmp")
    for tag, limit, cmd in _commands(name, out):
        print(f"[profile {name}] {tag}: {_display(cmd)}", flush=True)
        log = os.path.join(out, name, f"{tag}.log")
        os.makedirs(os.path.dirname(log), exist_ok=True)
        with open(log, "w") as f:
            r = subprocess.run(["timeout", "-s", "KILL", str(limit), *cmd], cwd="/tmp", env=env, stdout=f,
                               stderr=subprocess.STDOUT)
        print(f"[profile {name}] {tag}: exit {r.returncode}", flush=True)
        if r.returncode != 0:
            return r.returncode
    return 0


def _csv(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        return []
    with open(hits[0], newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def _match(kernel_name, key):
    return key in kernel_name


def _trace(d, kernels, timed):
    """Per kernel key: durations (us) of every dispatch in order, from the kernel trace."""
    rows = _csv(d, "kernel_trace.csv")
    out = {k: [] for k in kernels}
    rows.sort(key=lambda r: int(_col(r, "Start_Timestamp")))
    for r in rows:
        name = _col(r, "Kernel_Name")
        for k in kernels:
            if _match(name, k):
                out[k].append((int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3)
                break
    return out


def _counters(d, kernels):
    """Per kernel key: {counter: median per dispatch}, plus `_duration_ns` (median).  rocprofv3
    reports one value per dispatch and counter, summed over the hardware instances: the
    GRBM counters are then the sum over the eight XCDs."""
    rows = _csv(d, "counter_collection.csv")
    per = {k: {} for k in kernels}
    for r in rows:
        name = _col(r, "Kernel_Name")
        for k in kernels:
            if _match(name, k):
                disp = _col(r, "Dispatch_Id")
                per[k].setdefault(_col(r, "Counter_Name"), {})[disp] = float(_col(r, "Counter_Value"))
                per[k].setdefault("_duration_ns", {})[disp] = float(int(_col(r, "End_Timestamp")) -
                                                                     int(_col(r, "Start_Timestamp")))
                break
    return {k: {c: statistics.median(v.values()) for c, v in cs.items()} for k, cs in per.items()}


XCDS, CUS, SIMDS = 8, 256, 1024


def _load_traffic():
    try:
        with open(TRAFFIC) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def summarize(name, out):
    c = CASES[name]
    d = os.path.join(out, name)
    kernels = c["kernels"]
    lines = [f"# {c['title']}", "", "Commands (from the repository root, with TMPDIR=/tmp):"]
    lines += ["  " + _display(cmd) for _, _, cmd in _commands(name, "rocprof_out")]
    durs = _trace(os.path.join(d, "trace"), kernels, c["timed"])
    lines += ["", "Kernel durations from the kernel trace (microseconds):",
              f"  {'kernel':28s} {'dispatches':>10s} {'avg':>9s} {'min':>9s} {'max':>9s}   "
              f"{'last ' + str(c['timed']) + ' avg' if c['timed'] else ''}"]
    for k, v in durs.items():
        if not v:
            lines.append(f"  {k:28s} (no dispatch found)")
            continue
        last = v[-c["timed"]:] if c["timed"] else []
        tail = f"   {statistics.mean(last):9.1f}" if last else ""
        lines.append(f"  {k:28s} {len(v):10d} {statistics.mean(v):9.1f} {min(v):9.1f} {max(v):9.1f}{tail}")
    traffic = _load_traffic()
    cal = traffic.get("_calibration")
    fetch = _counters(os.path.join(d, "FETCH_SIZE"), kernels)
    write = _counters(os.path.join(d, "WRITE_SIZE"), kernels)
    if name == "hbm_copy":
        k = "copyBuffer"
        if "FETCH_SIZE" in fetch.get(k, {}) and "WRITE_SIZE" in write.get(k, {}):
            cal = {"fetch": (1 << 30) / (fetch[k]["FETCH_SIZE"] * 1024.0),
                   "write": (1 << 30) / (write[k]["WRITE_SIZE"] * 1024.0)}
            traffic["_calibration"] = dict(cal, source="profiles/hbm_copy.txt")
    lines += ["", "HBM-side counters, median per dispatch (KiB), scaled by the 1 GiB copy calibration"
              + (f" (FETCH x{cal['fetch']:.3f}, WRITE x{cal['write']:.3f}):" if cal else " (none yet):")]
    for k, (key, sources, algo, flop) in kernels.items():
        f_ = fetch.get(k, {}).get("FETCH_SIZE")
        w_ = write.get(k, {}).get("WRITE_SIZE")
        if f_ is None or w_ is None:
            continue
        line = f"  {k:28s} FETCH_SIZE {f_:12.1f}  WRITE_SIZE {w_:12.1f}"
        if cal:
            t = f_ * 1024.0 * cal["fetch"] + w_ * 1024.0 * cal["write"]
            line += f"  -> traffic {t / 1e6:10.1f} MB"
            if algo:
                line += f"  (algorithmic {algo / 1e6:.1f} MB, ratio {t / algo:.2f})"
            if key:
                traffic[key] = {"bytes": int(round(t)), "sources": sources, "source_sha": source_sha(sources),
                                "profile": f"profiles/{name}.txt"}
        lines.append(line)
    for i, counters in enumerate(c["pmc"]):
        cs = _counters(os.path.join(d, f"pmc{i + 1}"), kernels)
        lines += ["", f"Counter pass {i + 1}, median per dispatch: {' '.join(counters)}"]
        for k, v in cs.items():
            if not v:
                continue
            lines.append(f"  {k}:")
            for cn in counters:
                if cn in v:
                    lines.append(f"    {cn:28s} {v[cn]:16.0f}")
            g = v.get("GRBM_GUI_ACTIVE")
            if g:
                g /= XCDS                      # cycles per XCD: the kernel's length in shader cycles
                clk = (f"-> shader clock {g / v['_duration_ns']:.2f} GHz during this (serialised) dispatch"
                       if v["_duration_ns"] >= 200e3 else
                       "(dispatch too short for a clock estimate: the active span includes its start and drain)")
                lines.append(f"    GRBM_GUI_ACTIVE / {XCDS} XCDs = {g:.0f} cycles in {v['_duration_ns'] / 1e3:.1f} us {clk}")
            if g and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
                lines.append(f"    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {SIMDS} SIMDs) = "
                             f"{100 * v['SQ_VALU_MFMA_BUSY_CYCLES'] / (g * SIMDS):.1f} %")
            if v.get("SQ_LDS_IDX_ACTIVE"):
                lines.append(f"    LDS bank conflict / LDS active = "
                             f"{100 * v.get('SQ_LDS_BANK_CONFLICT', 0) / v['SQ_LDS_IDX_ACTIVE']:.1f} %")
            if g and "SQ_LDS_IDX_ACTIVE" in v:
                lines.append(f"    LDS active = SQ_LDS_IDX_ACTIVE / (cycles x {CUS} CUs) = "
                             f"{100 * v['SQ_LDS_IDX_ACTIVE'] / (g * CUS):.1f} %")
            if g and "SQ_ACTIVE_INST_VALU" in v:
                lines.append(f"    VALU active = SQ_ACTIVE_INST_VALU / (cycles x {SIMDS} SIMDs) = "
                             f"{100 * v['SQ_ACTIVE_INST_VALU'] / (g * SIMDS):.1f} %")
            if v.get("SQ_INSTS_MFMA") and flop:
                lines.append(f"    MFMA instructions per dispatch {v['SQ_INSTS_MFMA']:.0f} "
                             f"(expected {flop / 131072:.0f} of 32x32x64)")
    lines += ["", "FETCH_SIZE and WRITE_SIZE count requests between the L2 and the memory fabric, so reads",
              "served by the 256 MB Infinity Cache (MALL) are included.  Durations come from the same",
              "kind of run as the benchmark line (settle phase, warmup, timed steps); counter passes",
              "serialise dispatches and are not timed."]
    with open(os.path.join(PROFILES, f"{name}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(TRAFFIC, "w") as f:
        json.dump(traffic, f, indent=1, sort_keys=True)
        f.write("\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("action", choices=["run", "summarize", "list"])
    ap.add_argument("names", nargs="*")
    ap.add_argument("--out", default=os.path.join(ROOT, "rocprof_out"))
    a = ap.parse_args()
    if a.action == "list":
        print("\n".join(CASES))
        return 0
    for n in a.names:
        if n not in CASES:
            raise SystemExit(f"unknown profile {n}; one of {', '.join(CASES)}")
    for n in a.names:
        if a.action == "run":
            rc = run(n, a.out)
            if rc != 0:
                return rc
        else:
            summarize(n, a.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
