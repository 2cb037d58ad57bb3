"""Summaries of rocprofv3 runs of bench.py, written into profiles/.

    python bench_profiles.py trace   DIR             # DIR/run_kernel_stats.csv
    python bench_profiles.py traffic FETCH_DIR WRITE_DIR
    python bench_profiles.py sq      DIR             # DIR/run_counter_collection.csv
    python bench_profiles.py rates   FILE            # the JSON of bench.py --mfma-rates
    python bench_profiles.py crossover FILE          # the JSON of bench.py --crossover
    python bench_profiles.py lds     FILE            # the JSON of bench.py --lds-patterns

`trace` turns the --kernel-trace --stats summary of a bench run into
profiles/bench_kernel_trace.md.  `traffic` takes the two counter passes
(FETCH_SIZE, then WRITE_SIZE; each directory also holds bench.json, the JSON
line the profiled bench run printed), scales each counter by what it reads
for the plain 256 MiB copy that `bench.py --calib-copy` runs first, and
writes profiles/traffic.json (read by bench.py for `roofline.traffic`) and
profiles/hbm_counters.md.  `sq` writes the LDS and matrix-core counter table
profiles/lds_mfma_counters.md.  `rates` writes the sparse vs dense
matrix-core issue rates to profiles/mfma_rates_sparse_vs_dense.md, and
`crossover` the density study to profiles/crossover_fp16_8192x8192x16.md,
and `lds` the LDS read rates of per-lane address patterns to
profiles/lds_read_patterns.md.
Each summary names the command that made it;
COMMANDS below are those commands, run from the repository root of a GPU
machine with R set to that root.
"""
from __future__ import annotations

import csv
import json
import os
import re
import statistics
import sys

import bench

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")

COMMANDS = {
    "trace": "cd /tmp && timeout -k 10 900 rocprofv3 --kernel-trace --stats -f csv -d $R/gpurun_out/prof -o run "
             "-- python3 $R/bench.py --steps 20 --warmup 5 --no-cpu-baseline",
    "FETCH_SIZE": "mkdir -p $R/gpurun_out/pmc_FETCH_SIZE && cd /tmp && timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE -f csv -d $R/gpurun_out/pmc_FETCH_SIZE "
                  "-o run -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --only c2,c3,c5 "
                  "--workload-iters 10 --calib-copy > $R/gpurun_out/pmc_FETCH_SIZE/bench.json",
    "WRITE_SIZE": "mkdir -p $R/gpurun_out/pmc_WRITE_SIZE && cd /tmp && timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE -f csv -d $R/gpurun_out/pmc_WRITE_SIZE "
                  "-o run -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --only c2,c3,c5 "
                  "--workload-iters 10 --calib-copy > $R/gpurun_out/pmc_WRITE_SIZE/bench.json",
    "sq": "cd /tmp && timeout -s KILL 300 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
          "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_INSTS_MFMA SQ_WAVE_CYCLES SQ_WAVES GRBM_GUI_ACTIVE "
          "-f csv -d $R/gpurun_out/pmc_sq -o run -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline "
          "--only c2,c3,c5 --workload-iters 10",
    "rates": "mkdir -p $R/gpurun_out && timeout -k 10 120 python3 $R/bench.py --mfma-rates > $R/gpurun_out/mfma_rates.json",
    "crossover": "mkdir -p $R/gpurun_out && timeout -k 10 600 python3 $R/bench.py --crossover > $R/gpurun_out/crossover.json",
    "lds": "mkdir -p $R/gpurun_out && timeout -k 10 120 python3 $R/bench.py --lds-patterns > $R/gpurun_out/lds_patterns.json",
}

HEADLINE = "k_spmm_pipe<1, true, true, 8>"     # the headline step's product
TIMED = 20                                   # launches bench.py times back to back (--steps 20)

# Kernels the counter passes attribute to a workload line of bench.py:
# (kernel name as shortened below, workload line, kernel family, what).
# The workload line names the bench entry whose algorithmic bytes apply; the
# family names the sources whose hash marks the counters stale.
PROFILED = [
    ("k_spmm_pipe<1, true, true, 8>", "c4", "spmm_large_n",
     "bf16 28672x8192x2048 SpMM, packed prefill layout, B activation-major (the headline step's product)"),
    ("k_compress_prefill<1>", "c4", "compress",
     "bf16 28672x8192x2048 prune + compress into the packed prefill layout (the headline step's compress)"),
    ("k_spmm_pipe<1, true, false, 4>", "c4_bkn", "spmm_large_n",
     "bf16 28672x8192x2048 SpMM, packed prefill layout, B [K, N] row-major"),
    ("k_spmm_pipe<1, false, false, 4>", "c4_rowmajor", "spmm_large_n", "bf16 28672x8192x2048 SpMM, row-major operand"),
    ("k_spmm_pipe<2, true, true, 8>", "c2_prefill_bt", "spmm_large_n",
     "int8 4096^3 SpMM, packed prefill layout, B activation-major"),
    ("k_spmm_pipe<2, true, false, 4>", "c2_prefill", "spmm_large_n", "int8 4096^3 SpMM, packed prefill layout"),
    ("k_spmm_pipe<2, false, false, 4>", "c2", "spmm_large_n", "int8 4096^3 SpMM, row-major operand"),
    (re.compile(r"k_spmm_small_n_ring<0, \d+, \d+, false, false>"), "c3", "spmm_small_n",
     "fp16 11008x4096x16 SpMM, row-major operand"),
    (re.compile(r"k_spmm_packed<0, \d+, \d+, false, false, false>"), "c3_packed", "spmm_small_n",
     "fp16 11008x4096x16 SpMM, packed decode layout"),
    (re.compile(r"k_spmm_packed<0, \d+, \d+, false, false, true>"), "c3_packed_bt", "spmm_small_n",
     "fp16 11008x4096x16 SpMM, packed decode layout, B activation-major"),
    (re.compile(r"k_spmm_small_n_ring<0, \d+, \d+, true, false>"), "c5", "spmm_small_n",
     "fp16 8192x8192x16 2:4 + CSR residual, row-major operand"),
    (re.compile(r"k_spmm_small_n_ring<0, \d+, \d+, true, true>"), "c5_delta", "spmm_small_n",
     "fp16 8192x8192x16 2:4 + delta-coded residual, row-major operand"),
    (re.compile(r"k_spmm_packed<0, \d+, \d+, true, false, false>"), "c5_packed", "spmm_small_n",
     "fp16 8192x8192x16 2:4 + CSR residual, packed decode layout"),
    (re.compile(r"k_spmm_packed<0, \d+, \d+, true, true, false>"), "c5_delta_packed", "spmm_small_n",
     "fp16 8192x8192x16 2:4 + delta-coded residual, packed decode layout"),
    (re.compile(r"k_spmm_packed_cbm<0, \d+, \d+, false>"), "c5_cbm_packed", "spmm_small_n",
     "fp16 8192x8192x16 2:4 + complement-bitmap residual fused, packed decode layout"),
    (re.compile(r"k_spmm_packed_cbm<0, \d+, \d+, true>"), "c5_cbm_packed_bt", "spmm_small_n",
     "fp16 8192x8192x16 2:4 + complement-bitmap residual fused, packed decode layout, B activation-major"),
]


def short(name: str) -> str:
    """Readable kernel name: the library's template instantiation, the vendor
    GEMM's tile, or the first 100 characters."""
    if name.startswith("Cijk_"):
        t = re.search(r"Cijk_\w+?_(BBS|HHS|I8II|F8SS|SS|F8F8S\w*?)_", name)
        mt = re.search(r"_MT(\d+x\d+x\d+)_", name)
        return "vendor dense GEMM (%s, MT%s)" % (t.group(1) if t else "?", mt.group(1) if mt else "?")
    m = re.match(r"(?:void )?ssg::\(anonymous namespace\)::(\w+(?:<[^>]*>)?)", name)
    if m:
        return m.group(1)
    if "neg_kernel" in name:
        return "torch.neg (the 256 MiB copy reference)"
    return name[:100].replace("|", "/")


def match(kernel: str):
    for pat, line, family, what in PROFILED:
        if (pat == kernel) if isinstance(pat, str) else pat.fullmatch(kernel):
            return line, family, what
    return None


def header(title: str, cmds) -> str:
    s = "# %s\n\nCommand%s (from the repository root of the GPU machine, R = that root):\n\n```\n" % (
        title, "s" if len(cmds) > 1 else "")
    return s + "\n".join(cmds) + "\n```\n\n"


def trace(d: str) -> None:
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    out = [header("Kernel durations of the bench run (rocprofv3 --kernel-trace --stats)", [COMMANDS["trace"]]),
           "Every kernel of the default bench run without the CPU baseline: the headline step (bf16 28672x8192x2048, "
           "compress into the packed prefill layout + SpMM), the instruction-rate and streaming-read probes, and the "
           "workload table with the vendor dense GEMM of each shape.  Durations under the profiler run a few per cent "
           "longer than the HIP-event timings bench.py prints.\n\n",
           "| kernel | calls | avg us | min us | max us | total ms |\n|---|---|---|---|---|---|\n"]
    agg = {}
    for r in rows:
        k = short(r["Name"])
        a = agg.setdefault(k, [0, 0.0, float("inf"), 0.0])
        calls = int(r["Calls"])
        a[0] += calls
        a[1] += float(r["TotalDurationNs"])
        a[2] = min(a[2], float(r["MinNs"]))
        a[3] = max(a[3], float(r["MaxNs"]))
    for k, (calls, tot, mn, mx) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        out.append("| %s | %d | %.2f | %.2f | %.2f | %.2f |\n" % (k, calls, tot / calls / 1e3, mn / 1e3, mx / 1e3,
                                                                  tot / 1e6))
    # the headline product's last TIMED dispatches are the back-to-back
    # launches bench.py times with HIP events for roofline.launch_us
    tp = os.path.join(d, "run_kernel_trace.csv")
    if os.path.exists(tp):
        durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in csv.DictReader(open(tp))
                if short(r["Kernel_Name"]) == HEADLINE]
        last = durs[-TIMED:]
        if last:
            out.append("\nThe headline product %s: %d dispatches in the run; its last %d, the back-to-back launches "
                       "bench.py times with HIP events for `roofline.launch_us`, average %.2f us (min %.2f, max %.2f). "
                       "The other dispatches run inside the steps (after a compress) and in the graph check replays."
                       "\n" % (HEADLINE, len(durs), len(last), sum(last) / len(last) / 1e3, min(last) / 1e3,
                                max(last) / 1e3))
    with open(os.path.join(PROFILES, "bench_kernel_trace.md"), "w") as f:
        f.write("".join(out))


def counters(d: str):
    vals = {}
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        vals.setdefault(short(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    return vals


def bench_line(d: str) -> dict:
    with open(os.path.join(d, "bench.json")) as f:
        for line in f:
            if line.startswith("{"):
                return json.loads(line)
    raise SystemExit("no bench JSON line in %s/bench.json" % d)


def algorithmic_bytes(b: dict, line: str, family: str) -> int:
    if line in ("c4", "c4_bkn", "c4_rowmajor"):
        key = "compress_algorithmic_bytes_per_launch" if family == "compress" else "algorithmic_bytes_per_launch"
        return int(b["roofline"][key])
    return int(b["workloads"][line]["algorithmic_bytes_per_launch"])


def traffic(fetch_dir: str, write_dir: str) -> None:
    fe, wr = counters(fetch_dir), counters(write_dir)
    bl = bench_line(fetch_dir)
    ref = "torch.neg (the 256 MiB copy reference)"
    cf, cw = statistics.median(fe[ref]["FETCH_SIZE"]), statistics.median(wr[ref]["WRITE_SIZE"])
    fscale, wscale = 262144.0 / cf, 262144.0 / cw
    entries, table = {}, []
    for k in fe:
        m = match(k)
        if m is None or k not in wr:
            continue
        line, family, what = m
        f, w = statistics.median(fe[k]["FETCH_SIZE"]), statistics.median(wr[k]["WRITE_SIZE"])
        rb, wb = int(round(f * 1024 * fscale)), int(round(w * 1024 * wscale))
        ab = algorithmic_bytes(bl, line, family)
        entries["%s/%s" % (line, family)] = {
            "kernel": "%s (%s)" % (k, what), "kernel_source_sha": bench.kernel_source_sha(family),
            "FETCH_SIZE_KiB_per_dispatch": round(f, 1), "WRITE_SIZE_KiB_per_dispatch": round(w, 1),
            "dispatches": len(fe[k]["FETCH_SIZE"]),
            "fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5),
            "read_bytes_per_launch": rb, "write_bytes_per_launch": wb, "bytes_per_launch": rb + wb,
            "algorithmic_bytes_per_launch": ab}
        table.append((line, k, what, f, w, rb, wb, ab))
    doc = {"about": "HBM bytes per launch from rocprofv3 counters (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, "
                    "median over the run's dispatches, one pass each), scaled by what the same counters read for a "
                    "plain elementwise copy of 256 MiB (torch.neg on 64 Mi float32: reads 256 MiB, writes 256 MiB).",
           "commands": [COMMANDS["FETCH_SIZE"], COMMANDS["WRITE_SIZE"]],
           "copy_reference": {"FETCH_SIZE_KiB": round(cf, 1), "WRITE_SIZE_KiB": round(cw, 1),
                              "bytes_read": 268435456, "bytes_written": 268435456},
           "entries": dict(sorted(entries.items()))}
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    out = [header("HBM traffic of the profiled kernels (rocprofv3 FETCH_SIZE / WRITE_SIZE)",
                  [COMMANDS["FETCH_SIZE"], COMMANDS["WRITE_SIZE"]]),
           "FETCH_SIZE / WRITE_SIZE are KiB per dispatch, the median over the run's dispatches of the kernel.  "
           "Scale: the plain elementwise copy of 256 MiB reads FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB for "
           "262144 KiB each way, so reads scale by %.3f and writes by %.3f.  Algorithmic bytes: the unique bytes "
           "the kernel must move (compressed operand, B and C for a product; dense A in and packed operand out for "
           "the compress).\n\n" % (cf, cw, fscale, wscale),
           "| workload | kernel | what | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB | "
           "algorithmic MB | HBM / algorithmic |\n|---|---|---|---|---|---|---|---|---|\n"]
    for line, k, what, f, w, rb, wb, ab in sorted(table):
        out.append("| %s | %s | %s | %.1f | %.1f | %.1f | %.1f | %.1f | %.2f |\n" % (
            line, k, what, f, w, rb / 1e6, wb / 1e6, ab / 1e6, (rb + wb) / ab))
    with open(os.path.join(PROFILES, "hbm_counters.md"), "w") as f:
        f.write("".join(out))


def sq(d: str) -> None:
    c = counters(d)
    names = ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
             "SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
    out = [header("LDS and matrix-core counters of the profiled kernels (rocprofv3)", [COMMANDS["sq"]]),
           "Medians over each kernel's dispatches.  Conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (the "
           "cycles the LDS spends on bank conflicts over the cycles it is active).\n\n",
           "| kernel | what | " + " | ".join(names) + " | conflict share |\n|" + "---|" * (len(names) + 3) + "\n"]
    rows = []
    for k, cs in c.items():
        m = match(k)
        vendor = k.startswith("vendor dense GEMM")
        if m is None and not vendor:
            continue
        what = m[2] if m else "vendor dense GEMM of a profiled shape"
        med = {n: statistics.median(cs[n]) if n in cs else float("nan") for n in names}
        share = med["SQ_LDS_BANK_CONFLICT"] / med["SQ_LDS_IDX_ACTIVE"] if med["SQ_LDS_IDX_ACTIVE"] else 0.0
        rows.append((m[0] if m else "~", k, what, med, share))
    for _, k, what, med, share in sorted(rows, key=lambda r: (r[0], r[1])):
        out.append("| %s | %s | " % (k, what) + " | ".join("%.0f" % med[n] for n in names) + " | %.2f |\n" % share)
    with open(os.path.join(PROFILES, "lds_mfma_counters.md"), "w") as f:
        f.write("".join(out))


def rates(path: str) -> None:
    with open(path) as f:
        d = json.loads(f.read())
    forms = list(d["forms"].items())
    out = [header("Issue rates of the sparse and dense matrix-core instructions (the library's probe)",
                  [COMMANDS["rates"]]),
           "Dense-equivalent rate = 2 x rows x columns x dense k per instruction, over the launch (best of three), "
           "for one and two waves per SIMD (256 and 512 workgroups of four waves), random operands.  A sparse form "
           "covers twice the dense k of the dense form of the same tile (fp8: the dense 32x32x64 form covers the "
           "same k), so a kernel that decodes the 2:4 operand to dense and runs the dense form issues twice the "
           "instructions (fp8: the same number, at the dense form's rate) plus the decode.  Device: %s.\n\n"
           % d.get("device", "?"),
           "| sparse form | 1 wave/SIMD | 2 waves/SIMD | dense form | 1 wave/SIMD | 2 waves/SIMD | "
           "sparse / dense (1 wave) |\n|---|---|---|---|---|---|---|\n"]
    for (sn, sr), (dn, dr) in zip(forms[0::2], forms[1::2]):
        s1, s2 = sr["dense_equiv_rate_1_wave_per_simd"], sr["dense_equiv_rate_2_waves_per_simd"]
        d1, d2 = dr["dense_equiv_rate_1_wave_per_simd"], dr["dense_equiv_rate_2_waves_per_simd"]
        out.append("| %s | %.0f | %.0f | %s | %.0f | %.0f | %.2f |\n" % (sn, s1, s2, dn, d1, d2, s1 / d1))
    out.append("\nUnits: TFLOP/s for the floating-point forms, TOPS for int8.\n")
    with open(os.path.join(PROFILES, "mfma_rates_sparse_vs_dense.md"), "w") as f:
        f.write("".join(out))


def crossover(path: str) -> None:
    with open(path) as f:
        d = json.loads(f.read())
    out = [header("Unstructured sparsity vs dense vs 2:4 + residual: fp16 decode shape M=K=8192, N=16",
                  [COMMANDS["crossover"]]),
           "A is `randn * 0.02` kept with probability `density` (torch CUDA generator seeded 5000), rounded to "
           "fp16; B is `randn` [8192, 16] fp16.  Times are HIP events around back-to-back launches with >= 1 GiB of "
           "operand copies rotated.  dense = the vendor fp16 GEMM (torch.matmul) on A with its zeros; csr / delta = "
           "`ssg_spmm_csr` / `ssg_spmm_csr_delta` (no 2:4 layer); 2:4+CSR = `ssg_spmm_2to4_residual` on the exact "
           "split of A (residual epilogue); 2:4+bitmap = `ssg_spmm_2to4_packed_residual_cbm` on the same split, "
           "packed decode layout with the complement-bitmap residual fused into its k-steps.  Operand bytes are "
           "the sparse format's.\n\n",
           "| density | nnz | dense us | csr us | delta us | 2:4+CSR us | 2:4+bitmap us | csr MB | delta MB | "
           "2:4+CSR MB | 2:4+bitmap MB | max rel err vs fp32 |\n|" + "---|" * 12 + "\n"]
    for r in d["rows"]:
        out.append("| %.3f | %d | %.1f | %.1f | %.1f | %.1f | %.1f | %.1f | %.1f | %.1f | %.1f | %.1e |\n" % (
            r["density"], r["nnz"], r["dense_us"], r["csr_us"], r["delta_us"], r["split_us"], r["split_cbm_us"],
            r["csr_bytes"] / 1e6, r["delta_bytes"] / 1e6, r["split_bytes"] / 1e6, r["split_cbm_bytes"] / 1e6,
            r["max_rel_err_vs_fp32_dense"]))
    b = d["sparse_faster_than_dense_up_to_density"]
    out.append("\nSparse faster than dense up to density (of the densities measured): csr %s, delta %s, 2:4+CSR %s, "
               "2:4+bitmap %s.\n" % (b["csr"], b["delta"], b["split"], b["split_cbm"]))
    with open(os.path.join(PROFILES, "crossover_fp16_8192x8192x16.md"), "w") as f:
        f.write("".join(out))


def lds(path: str) -> None:
    with open(path) as f:
        d = json.loads(f.read())
    out = [header("LDS read rates of per-lane address patterns (the library's probe)", [COMMANDS["lds"]]),
           "One 16-byte read (ds_read_b128) per lane at the pattern's offset, eight reads 4 KiB apart in flight "
           "per wave, every value consumed; ns per read instruction per CU, best of three launches, at one and two "
           "workgroups of four waves per CU.  A read of 64 lanes moves 1 KiB.  Device: %s.\n\n" % d.get("device", "?"),
           "| pattern | 4 waves per CU | 8 waves per CU |\n|---|---|---|\n"]
    for r in d["patterns"]:
        out.append("| %s | %.2f | %.2f |\n" % (r["pattern"], r["ns_per_read_per_cu_4_waves"],
                                              r["ns_per_read_per_cu_8_waves"]))
    with open(os.path.join(PROFILES, "lds_read_patterns.md"), "w") as f:
        f.write("".join(out))


def main(argv) -> int:
    if len(argv) >= 2 and argv[0] == "trace":
        trace(argv[1])
    elif len(argv) >= 3 and argv[0] == "traffic":
        traffic(argv[1], argv[2])
    elif len(argv) >= 2 and argv[0] == "sq":
        sq(argv[1])
    elif len(argv) >= 2 and argv[0] == "rates":
        rates(argv[1])
    elif len(argv) >= 2 and argv[0] == "crossover":
        crossover(argv[1])
    elif len(argv) >= 2 and argv[0] == "lds":
        lds(argv[1])
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
