"""Benchmark of the 2:4 SpMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --mfma-rates      # sparse vs dense matrix-core issue rates
    python bench.py --lds-patterns    # LDS read rates of per-lane address patterns

Headline workload: the largest configuration, the bf16 prefill-shape 2:4
SpMM M=28672 K=8192 N=2048 (A ~ N(0, 0.02^2) magnitude-pruned 2:4 along K,
B ~ N(0, 1), fp32 accumulate).  One step is the whole hot path over one
batch: prune + compress A on the GPU straight into the packed prefill layout
(the large-N kernel's LDS image of each tile), then C = expand(packed) x B on
the large-N kernel, with the activations B handed over token-major (Bt =
B^T [N, K] row-major, as a linear layer's inputs arrive).  `value` is
dense-equivalent throughput 2*M*N*K / step time, inputs resident in HBM
before the timed region.  The same product with B [K, N] row-major, and with
the row-major (interchange) operand, are timed beside it.

Also printed, in the same JSON line:
* roofline: the SpMM kernel's own launch duration from HIP events recorded on
  the stream it runs on; achieved = algorithmic flops (M*N*K: two per stored
  non-zero product) / duration, against the dense bf16 MFMA peak; traffic
  from the committed rocprofv3 counter summary if it was taken on the current
  kernel source, else null; measured_instr_ceiling: the issue rate of the
  kernel's sparse MFMA form (and of the dense form a decode-to-dense kernel
  would issue) from the library's instruction probe;
* cpu_baseline: the CPU oracle (plain C, fp64) timed on this host on a
  bounded sample of rows of the same workload, checked against the GPU rows;
* oracle_baselines: the oracle on every configuration (single thread for the
  three small ones, all threads for the two large ones on row samples), with
  its compression / split timed apart from its product;
* workloads: kernel time and roofline fraction of the other shapes (small-N
  ones rotate >= 1 GiB of operand copies so the 256 MB Infinity Cache cannot
  serve repeated reads), each small-N line also against the measured
  streaming-read rate of the same number of bytes.
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

PEAK = {  # MI355X published peaks
    "hbm_GBps": 8000.0,
    "f16": 2516.6, "bf16": 2516.6, "i8": 5033.2,      # dense MFMA, TFLOP/s or TOPS
    "e4m3": 5033.2, "e5m2": 5033.2,
}
METRIC = "2:4 SpMM dense-equiv TFLOP/s (large N) and compressed-weight HBM GB/s (small N)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# source files that make up each profiled kernel (counters go stale when one changes)
KERNEL_SOURCES = {
    "spmm_large_n": ("spmm_large_n.hip", "ssg_device.hpp", "ssg_kernels.hpp"),
    "spmm_small_n": ("spmm_small_n.hip", "ssg_device.hpp", "ssg_kernels.hpp", "ssg_stream.hpp"),
    "spmm_nm": ("spmm_nm.hip", "ssg_device.hpp", "ssg_kernels.hpp", "ssg_stream.hpp"),
    "compress": ("compress.hip", "ssg_device.hpp", "ssg_kernels.hpp"),
}


def kernel_source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "structured_sparse_gemm_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get("entries", {}).get("%s/%s" % (workload, kernel))
    if not e or e.get("kernel_source_sha") != kernel_source_sha(kernel):
        return None
    return e.get("bytes_per_launch")


_ORACLE_DEFAULT_THREADS = {}


def cpu_baseline(w, a_cpu, b_cpu, target_s: float, threads: int = 0):
    """The oracle on the first R rows of the workload, R sized to about
    target_s of its product (all rows if they take less).  Compression (or the
    residual split) and the product are timed apart.  threads = 0: all host
    threads.  Returns the record and (rows, C, S) of the sample."""
    import oracle
    import workloads as W
    a, b = W.bits(a_cpu), W.bits(b_cpu)
    # all threads = the OpenMP default (OMP_NUM_THREADS where it is set)
    default = _ORACLE_DEFAULT_THREADS.setdefault("n", oracle.num_threads())
    oracle.set_num_threads(threads if threads > 0 else default)

    def run(rows):
        t0 = time.perf_counter()
        if w.residual:
            v, m, rp, col, rv = oracle.split(w.dtype, a[:rows])
            t1 = time.perf_counter()
            c, sb = oracle.spmm_residual(w.dtype, v, m, rp, col, rv, b, w.K)
        else:
            v, m = oracle.compress(w.dtype, a[:rows])
            t1 = time.perf_counter()
            c, sb = oracle.spmm(w.dtype, v, m, b, w.K)
        return t1 - t0, time.perf_counter() - t1, c, sb

    rows = min(w.M, 8)
    tc, tp, c, sb = run(rows)
    # grow the sample until its product takes about target_s (the first calls
    # are dominated by fixed costs such as converting B, so scale in steps)
    while tp < 0.5 * target_s and rows < w.M:
        rows = int(max(rows + 1, min(w.M, rows * min(8.0, 0.9 * target_s / max(tp, 1e-6)))))
        tc, tp, c, sb = run(rows)
    cores = oracle.num_threads()
    oracle.set_num_threads(default)
    return {
        "value": 2.0 * rows * w.N * w.K / tp / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "first %d of %d rows of A with all of B: product %.2f s (dense-equivalent rate), "
                  "%s %.2f s" % (rows, w.M, tp, "split" if w.residual else "prune/compress", tc),
        "product_seconds": tp,
        ("split_seconds" if w.residual else "compress_seconds"): tc,
        "rows": rows,
    }, (rows, c, sb)


def sample_matches(dtype: str, c_gpu, c_ref, s_ref) -> bool:
    """The GPU rows against the oracle's at the parity bar: int8 exact;
    floats relative Frobenius error <= 1e-3 and |err| <= 1e-2 * sum|a b|."""
    import numpy as np
    if dtype == "i8":
        return bool(np.array_equal(np.asarray(c_gpu).astype(np.int64), c_ref))
    c = np.asarray(c_gpu, dtype=np.float64)
    fro = np.linalg.norm(c - c_ref) / max(np.linalg.norm(c_ref), 1e-300)
    return bool(fro <= 1e-3 and (np.abs(c - c_ref) <= 1e-2 * s_ref).all())


def time_kernel(fn, iters: int, stream) -> float:
    """Average duration (s) of fn() launches, HIP events on `stream`."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(iters):
        fn(i)
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / iters


def graph_time(launches, reps: int, stream) -> float:
    """Average duration (s) of one launch: `launches` (a list of callables) is
    captured once into a HIP graph and replayed `reps` times between two HIP
    events on `stream`."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in launches:
            f()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * len(launches))


_READ_BW = {}


def read_bandwidth_GBps(nbytes: int, reps: int = 2) -> float:
    """Achievable read rate (GB/s) for a stream of nbytes: the library's
    streaming-read probe over copies of that size rotated through >= 1 GiB
    (so the Infinity Cache serves no repeated read), launched like the
    workloads (one HIP graph of back-to-back launches)."""
    import numpy as np
    import torch

    import structured_sparse_gemm_amd as ssg
    nbytes = max(16, (int(nbytes) + 15) // 16 * 16)
    if nbytes in _READ_BW:
        return _READ_BW[nbytes]
    copies = max(2, int(np.ceil((1 << 30) / nbytes)))
    bufs = [torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
    sink = torch.zeros(max(1, ssg.ssg_stream_read_sink_words(nbytes)), dtype=torch.int32, device="cuda")
    n = max(copies, 50)
    s = graph_time([lambda i=i: ssg.ssg_stream_read(bufs[i % copies], sink) for i in range(n)], reps,
                   torch.cuda.current_stream())
    del bufs, sink
    torch.cuda.empty_cache()
    _READ_BW[nbytes] = nbytes / s / 1e9
    return _READ_BW[nbytes]


_MFMA = {}


def mfma_rate(form: int, per_cu: int = 1, iters: int = 2000, reps: int = 3) -> float:
    """Dense-equivalent rate (TFLOP/s or TOPS) of one matrix-core instruction
    form: the library's issue-rate probe on per_cu workgroups of four waves
    per CU (one wave per SIMD for per_cu = 1), best of `reps` launches timed
    with HIP events on the current stream."""
    import torch

    import structured_sparse_gemm_amd as ssg
    if (form, per_cu, iters) in _MFMA:
        return _MFMA[(form, per_cu, iters)]
    wg = per_cu * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(wg, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ssg.ssg_mfma_probe(form, wg, 10, sink)                   # warm-up
    best = min(time_kernel(lambda i: ssg.ssg_mfma_probe(form, wg, iters, sink), 1, stream) for _ in range(reps))
    _MFMA[(form, per_cu, iters)] = ssg.ssg_mfma_probe_ops(form, wg, iters) / best / 1e12
    return _MFMA[(form, per_cu, iters)]


def mfma_rates() -> dict:
    """Every form of the probe at one and two workgroups per CU."""
    import structured_sparse_gemm_amd as ssg
    return {ssg.ssg_mfma_probe_name(f): {"dense_equiv_rate_1_wave_per_simd": mfma_rate(f, 1),
                                         "dense_equiv_rate_2_waves_per_simd": mfma_rate(f, 2)}
            for f in range(ssg.ssg_mfma_probe_forms())}


def lds_patterns() -> list:
    """Per-lane address patterns of one 16-byte LDS read (64 byte offsets,
    one per lane): the contiguous read, pairs of lanes k apart on one bank
    at different addresses, and the reads of the large-N kernel's LDS images
    (two row images of the sparse values, the lane-ordered one the packed
    prefill layout gives, and the activation-major B tile with and without
    its swizzle)."""
    def swz_rows(r):
        return ((r >> 1) ^ (r >> 3)) & 3

    pats = [("contiguous (lane l at 16 l)", [16 * l for l in range(64)])]
    for k in (1, 2, 4, 8, 16, 32):
        pats.append(("lanes l and l+%d on one bank, 1 KiB apart" % k,
                     [16 * (l - k) + 1024 if l & k else 16 * l for l in range(64)]))
    pats.append(("sparse values, rows of 64 B, chunks swizzled by ((r/2)^(r/8))%4",
                 [(l & 31) * 64 + (((l >> 5) ^ swz_rows(l & 31)) << 4) for l in range(64)]))
    pats.append(("the same, lanes 0-15 only (the rest contiguous, 8 KiB on)",
                 [(l & 31) * 64 + (((l >> 5) ^ swz_rows(l & 31)) << 4) if l < 16 else 8192 + 16 * l
                  for l in range(64)]))
    pats.append(("sparse values, rows of 64 B, chunks swizzled by (r/4)%2 + 2((r^r/16)%2) (row-major operand)",
                 [(l & 31) * 64 + (((l >> 5) ^ (((l & 31) >> 2) & 1) ^ ((((l & 31) ^ ((l & 31) >> 4)) & 1) << 1)) << 4)
                  for l in range(64)]))
    pats.append(("sparse values, rows of 64 B, unswizzled", [(l & 31) * 64 + ((l >> 5) << 4) for l in range(64)]))
    pats.append(("sparse values, packed prefill layout (lane order)", [16 * l for l in range(64)]))
    pats.append(("activation-major B, rows of 128 B, chunks swizzled by (n/2)%8",
                 [(l & 31) * 128 + (((l >> 5) ^ ((l & 31) >> 1 & 7)) << 4) for l in range(64)]))
    pats.append(("activation-major B, rows of 128 B, unswizzled", [(l & 31) * 128 + ((l >> 5) << 4) for l in range(64)]))
    pats.append(("the 16 lanes of each group on one bank, 256 B apart", [256 * (l & 15) for l in range(64)]))
    return pats


def lds_read_rates(iters: int = 2000, reps: int = 3) -> list:
    """ns per 16-byte read instruction per CU for each pattern of
    lds_patterns(), at one and two workgroups of four waves per CU, best of
    `reps` launches timed with HIP events on the current stream."""
    import torch

    import structured_sparse_gemm_amd as ssg
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sink = torch.zeros(2 * cus, dtype=torch.int32, device="cuda")
    pats = lds_patterns()
    for _ in range(3):                                           # clocks up before the first timing
        ssg.ssg_lds_read_probe(pats[0][1], 2 * cus, iters, sink)
    out = []
    for name, offs in pats:
        row = {"pattern": name}
        for per_cu in (1, 2):
            wg = per_cu * cus
            ssg.ssg_lds_read_probe(offs, wg, 10, sink)             # warm-up
            best = min(time_kernel(lambda i: ssg.ssg_lds_read_probe(offs, wg, iters, sink), 1, stream)
                       for _ in range(reps))
            row["ns_per_read_per_cu_%d_waves" % (4 * per_cu)] = best * 1e9 / (per_cu * 4 * 8 * iters)
        out.append(row)
    return out


def bench_workload(key: str, iters: int, delta: bool = False, dense_cmp: bool = True,
                   packed: bool = False, nm=None, prefill: bool = False, cbm: bool = False, bt: bool = False):
    """Kernel-level numbers for one workload (compression outside the timing),
    next to a dense GEMM of the same shape from the vendor library.  With
    delta=True the residual is delta-coded (one-byte column gaps); with
    packed=True the 2:4 operand is in the packed decode layout; with
    prefill=True in the packed prefill layout (bt=True, with prefill or
    packed: B handed over activation-major, as Bt [N, K] row-major); with
    nm=(n, m) the weight is
    in the n:m form (kept values plus keep mask); with cbm=True (and packed)
    the residual is in the complement-bitmap layout, fused into the packed
    product's k-steps."""
    import numpy as np
    import torch

    import structured_sparse_gemm_amd as ssg
    import workloads as W
    w = W.WORKLOADS[key]
    a = W.gen_a(w).cuda()
    b = W.gen_b(w).cuda()
    b_t = b.t().contiguous() if bt else None
    if nm is not None:
        ops = ssg.compress_nm(a, nm[0], nm[1])
        if packed:
            ops = ssg.pack_nm(ops[0], ops[1], nm[0], nm[1], w.K)
    elif prefill:
        ops = ssg.compress_prefill(a)
    else:
        ops = ssg.split(a) if w.residual else ssg.compress(a)
    if delta:
        ops = ops[:2] + ssg.delta_encode(ops[2], ops[3], ops[4], w.K)
    if packed and nm is None:
        ops = ssg.pack_decode(ops[0], ops[1], w.K) + tuple(ops[2:])
    if cbm:
        vals0, meta0, rp0, col0, rv0 = ssg.split(a)
        pv0, pm0 = ssg.pack_decode(vals0, meta0, w.K)
        ops = (pv0, pm0) + ssg.pack_residual_cbm(meta0, rp0, col0, rv0, w.K)
        del vals0, meta0, rp0, col0, rv0
    wbytes = sum(t.numel() * t.element_size() for t in ops)
    copies = 1
    if w.klass == "small_n":
        copies = max(1, int(np.ceil((1 << 30) / wbytes)))
    sets = [ops] + [tuple(t.clone() for t in ops) for _ in range(copies - 1)]
    out = torch.empty((w.M, w.N), dtype=torch.int32 if w.dtype == "i8" else torch.float32, device="cuda")
    algo = (ssg.SSG_ALGO_SMALL_N if packed or nm else ssg.SSG_ALGO_LARGE_N if prefill
            else ssg.ssg_spmm_select_algo(ops[0], ops[1], b, out))

    def launch(i):
        o = sets[i % copies]
        if cbm and bt:
            ssg.ssg_spmm_2to4_packed_residual_cbm_bt(o[0], o[1], w.M, o[2], o[3], o[4], b_t, out)
        elif cbm:
            ssg.ssg_spmm_2to4_packed_residual_cbm(o[0], o[1], w.M, o[2], o[3], o[4], b, out)
        elif nm is not None and packed:
            ssg.ssg_spmm_nm_packed(o[0], o[1], nm[0], nm[1], w.M, b, out, i4=w.dtype == "i4")
        elif nm is not None:
            ssg.ssg_spmm_nm(o[0], o[1], nm[0], nm[1], w.K, b, out)
        elif packed and delta:
            ssg.ssg_spmm_2to4_packed_residual_delta(o[0], o[1], w.M, o[2], o[3], o[4], b, out)
        elif packed and w.residual:
            ssg.ssg_spmm_2to4_packed_residual(o[0], o[1], w.M, o[2], o[3], o[4], b, out)
        elif packed and bt:
            ssg.ssg_spmm_2to4_packed_bt(o[0], o[1], w.M, b_t, out)
        elif packed:
            ssg.ssg_spmm_2to4_packed(o[0], o[1], w.M, b, out)
        elif prefill and bt:
            ssg.ssg_spmm_2to4_prefill_bt(o[0], o[1], w.M, b_t, out)
        elif prefill:
            ssg.ssg_spmm_2to4_prefill(o[0], o[1], w.M, b, out)
        elif delta:
            ssg.ssg_spmm_2to4_residual_delta(*o, b, out)
        elif w.residual:
            ssg.ssg_spmm_2to4_residual(*o, b, out)
        else:
            ssg.ssg_spmm_2to4(o[0], o[1], b, out)

    stream = torch.cuda.current_stream()
    n = max(iters, copies)
    for i in range(n):
        launch(i)
    torch.cuda.synchronize()
    ref = out.clone()                                   # eager result of the last launch
    s = graph_time([lambda i=i: launch(i) for i in range(n)], 2, stream)
    graph_ok = bool(torch.equal(out, ref))
    flops = 2.0 * w.M * w.N * w.K
    bbytes = b.numel() * b.element_size()
    cbytes = out.numel() * out.element_size()
    tkey = key + ("_%d:%d" % tuple(nm) if nm else "") + ("_delta" if delta else "") + ("_cbm" if cbm else "") \
        + ("_packed" if packed else "") + ("_prefill" if prefill else "") + ("_bt" if bt else "")
    family = "spmm_nm" if nm else "spmm_large_n" if w.klass == "large_n" else "spmm_small_n"
    r = {"title": w.title + (", residual delta-coded" if delta else "") + (", packed decode layout" if packed else "")
         + (", complement-bitmap residual fused" if cbm else "")
         + (", packed prefill layout" if prefill else "") + (", B activation-major (Bt [N, K])" if bt else "")
         + (", %d:%d" % tuple(nm) if nm else ""),
         "algo": ("nm (dense MFMA on the expanded operand)" if nm else ssg.ALGO_NAMES[algo])
         + (" (packed)" if packed else "") + (" (packed prefill)" if prefill else ""),
         "us_per_launch": s * 1e6,
         "timing": "HIP graph of %d launches, replayed twice; replay output matches eager: %s" % (n, graph_ok),
         "dense_equiv_TFLOPs": flops / s / 1e12, "compressed_weight_bytes": wbytes,
         "algorithmic_bytes_per_launch": wbytes + bbytes + cbytes,
         "compressed_weight_GBps": wbytes / s / 1e9, "operand_copies_rotated": copies}
    if w.klass == "large_n":
        r["frac_dense_peak"] = flops / s / 1e12 / PEAK[w.dtype]
        r["frac_sparse_peak"] = r["frac_dense_peak"] / 2
        # roofline of the kernel: algorithmic ops (two per stored product) over
        # the launch duration, against the dense MFMA peak of the dtype
        r["roofline"] = {"bound": "mfma", "achieved": flops / 2 / s / 1e12, "peak": PEAK[w.dtype],
                         "unit": "TFLOP/s", "frac": flops / 2 / s / 1e12 / PEAK[w.dtype],
                         "traffic": traffic_for(tkey, family)}
    else:
        r["frac_hbm_weights"] = wbytes / s / 1e9 / PEAK["hbm_GBps"]
        r["frac_hbm_all_bytes"] = (wbytes + bbytes + cbytes) / s / 1e9 / PEAK["hbm_GBps"]
        # roofline of the kernel: the bytes it must move (compressed weights,
        # B, C) over the launch duration, against the HBM peak
        r["roofline"] = {"bound": "hbm", "achieved": (wbytes + bbytes + cbytes) / s / 1e9, "peak": PEAK["hbm_GBps"],
                         "unit": "GB/s", "frac": (wbytes + bbytes + cbytes) / s / 1e9 / PEAK["hbm_GBps"],
                         "traffic": traffic_for(tkey, family)}
        rbw = read_bandwidth_GBps(wbytes)
        r["measured_read_GBps_same_bytes"] = rbw
        r["frac_measured_read_bw_weights"] = wbytes / s / 1e9 / rbw
    del sets, ops, out
    torch.cuda.empty_cache()
    if not dense_cmp:
        return r

    # dense comparator: the same product as a dense GEMM (vendor library via
    # torch), weights as a dense matrix, copies rotated like the sparse ones;
    # for 4-bit weights, dense fp16 weights of the same shape
    dense = a if w.dtype != "i4" else (torch.randn((w.M, w.K), device="cuda") * 0.02).half()
    dbytes = dense.numel() * dense.element_size()
    dcopies = max(1, int(np.ceil((1 << 30) / dbytes))) if w.klass == "small_n" else 1
    dsets = [dense] + [dense.clone() for _ in range(dcopies - 1)]
    del a
    if w.dtype == "i8":
        dfn = lambda x: torch._int_mm(x, b)
    elif w.dtype in ("e4m3", "e5m2"):
        # the vendor fp8 GEMM through torch: unit scales, B column-major, fp32 out
        one = torch.ones((), dtype=torch.float32, device="cuda")
        bt = b.t().contiguous().t()
        dfn = lambda x: torch._scaled_mm(x, bt, scale_a=one, scale_b=one, out_dtype=torch.float32)
    else:
        dfn = lambda x: torch.matmul(x, b)
    nd = max(iters, dcopies)
    try:
        for i in range(nd):
            dfn(dsets[i % dcopies])
        torch.cuda.synchronize()
        sd = time_kernel(lambda i: dfn(dsets[i % dcopies]), nd, stream)
        r["dense_gemm_us"] = sd * 1e6
        r["dense_gemm"] = "torch %s on dense weights of the same shape (%s output), back-to-back launches" % (
            {"i8": "_int_mm", "e4m3": "_scaled_mm", "e5m2": "_scaled_mm"}.get(w.dtype, "matmul"),
            {"i8": "int32", "e4m3": "fp32", "e5m2": "fp32"}.get(w.dtype, w.dtype))
        r["speedup_vs_dense"] = sd / s
    except RuntimeError as e:
        r["dense_gemm"] = "unavailable: %s" % str(e).splitlines()[0][:120]
    del dsets, dense, b
    torch.cuda.empty_cache()
    return r


def crossover(iters: int) -> dict:
    """Unstructured sparsity against dense and 2:4 at the fp16 decode shape
    M = K = 8192, N = 16: for each density, the vendor dense GEMM on the
    matrix with its zeros, the plain CSR and delta-coded sparse products,
    and the exact 2:4 + residual split of the same matrix (CSR residual
    epilogue, and the complement-bitmap residual fused into the packed
    product).  Operand copies
    (>= 1 GiB) are rotated so the Infinity Cache serves no repeated reads."""
    import numpy as np
    import torch

    import structured_sparse_gemm_amd as ssg
    M = K = 8192
    N = 16
    g = torch.Generator(device="cuda")
    g.manual_seed(5000)
    B = torch.randn((K, N), generator=g, device="cuda").half()
    stream = torch.cuda.current_stream()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def timed(base, launch):
        nbytes = sum(t.numel() * t.element_size() for t in base)
        copies = max(1, int(np.ceil((1 << 30) / nbytes)))
        sets = [base] + [tuple(t.clone() for t in base) for _ in range(copies - 1)]
        n = max(iters, copies)
        for i in range(n):
            launch(sets[i % copies])
        torch.cuda.synchronize()
        t = time_kernel(lambda i: launch(sets[i % copies]), n, stream)
        del sets
        torch.cuda.empty_cache()
        return t * 1e6, nbytes

    rows = []
    for d in (0.002, 0.005, 0.01, 0.02, 0.05, 0.1, 0.2, 0.3, 0.5):
        A = torch.randn((M, K), generator=g, device="cuda") * 0.02
        A = torch.where(torch.rand((M, K), generator=g, device="cuda") < d, A, torch.zeros((), device="cuda"))
        A = A.half()
        nz = A.nonzero()                                   # row-major order: columns ascend within a row
        row_ptr = torch.zeros(M + 1, dtype=torch.int32, device="cuda")
        row_ptr[1:] = torch.cumsum(torch.bincount(nz[:, 0], minlength=M), 0).int()
        col = nz[:, 1].int().contiguous()
        vals = A[nz[:, 0], nz[:, 1]].contiguous()
        del nz
        dl = ssg.delta_encode(row_ptr, col, vals, K)
        sp = ssg.split(A)
        ref = A.float() @ B.float()
        r = {"density": d, "nnz": int(col.numel()), "delta_entries": int(dl[1].numel())}
        r["dense_us"], r["dense_bytes"] = timed((A,), lambda o: torch.matmul(o[0], B))
        r["csr_us"], r["csr_bytes"] = timed((row_ptr, col, vals), lambda o: ssg.ssg_spmm_csr(*o, B, out))
        err_csr = float((out - ref).abs().max() / ref.abs().max())
        r["delta_us"], r["delta_bytes"] = timed(dl, lambda o: ssg.ssg_spmm_csr_delta(*o, B, out))
        err_delta = float((out - ref).abs().max() / ref.abs().max())
        r["split_us"], r["split_bytes"] = timed(sp, lambda o: ssg.ssg_spmm_2to4_residual(*o, B, out))
        err_split = float((out - ref).abs().max() / ref.abs().max())
        # the same split with the residual as a complement bitmap, fused into
        # the packed decode product's k-steps
        cb = ssg.pack_decode(sp[0], sp[1], K) + ssg.pack_residual_cbm(sp[1], sp[2], sp[3], sp[4], K)
        r["split_cbm_us"], r["split_cbm_bytes"] = timed(
            cb, lambda o: ssg.ssg_spmm_2to4_packed_residual_cbm(o[0], o[1], M, o[2], o[3], o[4], B, out))
        err_cbm = float((out - ref).abs().max() / ref.abs().max())
        r["max_rel_err_vs_fp32_dense"] = max(err_csr, err_delta, err_split, err_cbm)
        rows.append(r)
        print("crossover: density %.3f: dense %.1f us, csr %.1f us, delta %.1f us, 2:4+residual %.1f us, "
              "2:4+bitmap fused %.1f us" % (d, r["dense_us"], r["csr_us"], r["delta_us"], r["split_us"],
                                            r["split_cbm_us"]), file=sys.stderr, flush=True)
        del A, row_ptr, col, vals, dl, sp, cb, ref
        torch.cuda.empty_cache()

    def below(key):
        ok = [r["density"] for r in rows if r[key] < r["dense_us"]]
        return max(ok) if ok else None
    return {"study": "unstructured sparsity vs dense vs 2:4 at the fp16 decode shape M=K=8192, N=16",
            "timing": "HIP events around back-to-back launches, >= 1 GiB of operand copies rotated",
            "rows": rows,
            "sparse_faster_than_dense_up_to_density": {"csr": below("csr_us"), "delta": below("delta_us"),
                                                        "split": below("split_us"),
                                                        "split_cbm": below("split_cbm_us")}}


def main() -> int:
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample size, in seconds of CPU work")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-oracle-table", action="store_true", help="skip the oracle timings of the other configs")
    p.add_argument("--no-workloads", action="store_true", help="skip the per-workload table")
    p.add_argument("--workload-iters", type=int, default=0,
                   help="launches per workload in the table (default 200 for small N, 20 for large N)")
    p.add_argument("--calib-copy", action="store_true",
                   help="first run a plain elementwise copy of 256 MiB (read 256 MiB, write 256 MiB) three times, "
                        "outside the timed region: the reference for scaling HBM byte counters")
    p.add_argument("--only", default="", help="comma-separated workload keys of the table (default: all)")
    p.add_argument("--lds-patterns", action="store_true",
                   help="print the LDS read rate of each per-lane address pattern and exit")
    p.add_argument("--mfma-rates", action="store_true",
                   help="instead of the benchmark, print the issue rates of the sparse and dense matrix-core "
                        "instruction forms (the library's probe) as JSON")
    p.add_argument("--crossover", action="store_true",
                   help="instead of the benchmark, run the unstructured-sparsity crossover study and print its JSON")
    args = p.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus %d)" % args.gpus,
              file=sys.stderr)
        return 2

    import torch

    import structured_sparse_gemm_amd as ssg
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm device", file=sys.stderr)
        return 1

    if args.crossover:
        print(json.dumps(crossover(args.workload_iters or 100)))
        return 0

    if args.mfma_rates:
        print(json.dumps({"unit": "dense-equivalent TFLOP/s (TOPS for int8)", "forms": mfma_rates(),
                          "device": torch.cuda.get_device_name(0)}))
        return 0

    if args.lds_patterns:
        print(json.dumps({"unit": "ns per 16-byte read instruction per CU", "patterns": lds_read_rates(),
                          "device": torch.cuda.get_device_name(0)}))
        return 0

    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    key = "c4"
    w = W.WORKLOADS[key]
    print("bench: %s" % w.title, file=sys.stderr, flush=True)
    a_cpu, b_cpu = W.gen_a(w), W.gen_b(w)
    A, B = a_cpu.cuda(), b_cpu.cuda()
    vb, mb = ssg.ssg_prefill_packed_sizes(A.dtype, w.M, w.K)
    vals = torch.empty(vb, dtype=torch.uint8, device="cuda")       # packed prefill layout
    meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
    out_dt = torch.int32 if w.dtype == "i8" else torch.float32
    C = torch.empty((w.M, w.N), dtype=out_dt, device="cuda")
    stream = torch.cuda.current_stream()

    # the activations handed over token-major, Bt = B^T [N, K] row-major, as
    # a linear layer's inputs arrive (prepared before the timed region)
    Bt = B.t().contiguous()

    def step():
        ssg.ssg_compress_2to4_prefill(A, vals, meta)
        ssg.ssg_spmm_2to4_prefill_bt(vals, meta, w.M, Bt, C)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref_vals, ref_meta, ref_C = vals.clone(), meta.clone(), C.clone()

    # The K timed steps are captured once into one HIP graph (each step its
    # full compress + SpMM, 2K kernel nodes) and replayed once, so the host
    # pays one graph launch for the K steps instead of one per step.  Each
    # check replay follows eager work and a synchronisation and must
    # reproduce the eager outputs bit for bit.
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()
    graph_ok = True
    for _ in range(3):
        vals.zero_(); meta.zero_(); C.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        graph_ok &= bool(torch.equal(vals, ref_vals) and torch.equal(meta, ref_meta) and
                         torch.equal(C.view(torch.int32), ref_C.view(torch.int32)))
        step()
        torch.cuda.synchronize()
    del ref_vals, ref_meta

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    del graph

    # kernel durations: back-to-back launches between two HIP events on the
    # stream the kernels run on
    reps = max(args.steps, 20)
    spmm_s = time_kernel(lambda i: ssg.ssg_spmm_2to4_prefill_bt(vals, meta, w.M, Bt, C), reps, stream)
    comp_s = time_kernel(lambda i: ssg.ssg_compress_2to4_prefill(A, vals, meta), reps, stream)
    # the same product with B [K, N] row-major
    C_kn = torch.empty_like(C)
    ssg.ssg_spmm_2to4_prefill(vals, meta, w.M, B, C_kn)
    torch.cuda.synchronize()
    b_rowmajor = {"spmm_us": time_kernel(lambda i: ssg.ssg_spmm_2to4_prefill(vals, meta, w.M, B, C_kn), reps,
                                         stream) * 1e6,
                  "same_result_bits": bool(torch.equal(C_kn.view(torch.int32), C.view(torch.int32)))}
    del C_kn
    # the same product from the row-major (interchange) operand
    rvals, rmeta = ssg.compress(A)
    C_rm = ssg.spmm(rvals, rmeta, B, algo=ssg.SSG_ALGO_LARGE_N)
    torch.cuda.synchronize()
    rowmajor = {"spmm_us": time_kernel(lambda i: ssg.ssg_spmm_2to4(rvals, rmeta, B, C_rm), reps, stream) * 1e6,
                "same_result_bits": bool(torch.equal(C_rm.view(torch.int32), C.view(torch.int32)))}
    del rvals, rmeta, C_rm
    torch.cuda.empty_cache()
    flops = 2.0 * w.M * w.N * w.K
    algo_ops = float(w.M) * w.N * w.K          # two per stored product, half the positions stored
    print("bench: step %.3f ms (graph replay; compress %.1f us, spmm %.1f us)" % (ms, comp_s * 1e6, spmm_s * 1e6),
          file=sys.stderr, flush=True)

    dense_note = None
    try:
        torch.matmul(A, B)
        torch.cuda.synchronize()
        dense_s = time_kernel(lambda i: torch.matmul(A, B), reps, stream)
        dense_note = {"dense_gemm_us": dense_s * 1e6, "speedup_spmm_vs_dense": dense_s / spmm_s,
                      "dense_gemm": "torch matmul (bf16 x bf16 -> bf16, vendor library) on the dense weights, "
                                    "back-to-back launches"}
    except RuntimeError as e:
        dense_note = {"dense_gemm": "unavailable: %s" % str(e).splitlines()[0][:120]}
    torch.cuda.empty_cache()

    roofline = {
        "kernel": "spmm_large_n on the packed prefill layout, B activation-major (bf16 sparse MFMA 32x32x32)",
        "bound": "mfma",
        "achieved": algo_ops / spmm_s / 1e12,
        "peak": PEAK[w.dtype],
        "unit": "TFLOP/s",
        "frac": algo_ops / spmm_s / 1e12 / PEAK[w.dtype],
        "traffic": traffic_for(key, "spmm_large_n"),
        "launch_us": spmm_s * 1e6,
        "dense_equiv_frac_of_dense_peak": flops / spmm_s / 1e12 / PEAK[w.dtype],
        "algorithmic_flops_per_launch": algo_ops,
        # unique bytes the product must move: the packed operand, B, C
        "algorithmic_bytes_per_launch": vb + mb + B.numel() * B.element_size() + C.numel() * C.element_size(),
        "compress_algorithmic_bytes_per_launch": A.numel() * A.element_size() + vb + mb,
        "compress_traffic": traffic_for(key, "compress"),
    }
    # the measured issue rate of the kernel's instruction (and of the dense
    # form a decode-to-dense kernel would issue instead), one wave per SIMD
    sp, de = mfma_rate(0), mfma_rate(1)
    roofline["measured_instr_ceiling"] = {
        "instr": ssg.ssg_mfma_probe_name(0), "algorithmic_TFLOPs": sp / 2, "dense_equiv_TFLOPs": sp,
        "frac": algo_ops / spmm_s / 1e12 / (sp / 2),
        "dense_instr": ssg.ssg_mfma_probe_name(1), "dense_instr_TFLOPs": de}
    out = {
        "metric": METRIC,
        "value": flops / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": "bf16 2:4 SpMM M=28672 K=8192 N=2048 (prefill shape); step = prune+compress A "
                               "(packed prefill layout), then SpMM with the activations B handed over "
                               "token-major (Bt [N, K] row-major), fp32 out",
                   "M": w.M, "K": w.K, "N": w.N, "seeds": [1000 + w.index, 2000 + w.index]},
        "spmm_only_dense_equiv_TFLOPs": flops / spmm_s / 1e12,
        "spmm_us": spmm_s * 1e6,
        "compress_us": comp_s * 1e6,
        "b_kn_rowmajor": b_rowmajor,
        "rowmajor_operand": rowmajor,
        "launch": "one HIP graph of the %d timed steps (each: compress + SpMM), replayed once; check replays "
                  "match eager outputs: %s" % (args.steps, graph_ok),
        "device": "%s, HIP %s" % (torch.cuda.get_device_name(0), torch.version.hip),
        "roofline": roofline,
        "dense_comparator": dense_note,
    }
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cb, (rows, cref, sref) = cpu_baseline(w, a_cpu, b_cpu, args.cpu_seconds)
        cb["sample_matches_gpu"] = sample_matches(w.dtype, C[:rows].cpu().numpy(), cref, sref)
        out["cpu_baseline"] = cb
    del A, B, vals, meta, C, a_cpu, b_cpu
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and not args.no_oracle_table:
        # the oracle on every configuration: one thread for the three small
        # ones (whole), all threads on row samples of the two large ones
        table = {}
        for k, threads, secs in (("c1", 1, 1.0), ("c3", 1, 3.0), ("c5", 1, 3.0), ("c2", 0, 3.0)):
            wk = W.WORKLOADS[k]
            print("bench: oracle on %s ..." % k, file=sys.stderr, flush=True)
            rec, _ = cpu_baseline(wk, W.gen_a(wk), W.gen_b(wk), secs, threads=threads)
            table[k] = rec
        table["c4"] = {kk: vv for kk, vv in out.get("cpu_baseline", {}).items()}
        out["oracle_baselines"] = table
    if not args.no_workloads:
        out["measured_read_GBps_1GiB"] = read_bandwidth_GBps(1 << 30)
        table = {}
        only = [k for k in args.only.split(",") if k]
        for k in ("c1", "c2", "c3", "c4", "c5", "c3f8", "c4f8", "c3nm", "c3w4"):
            if only and k not in only:
                continue
            if k in ("c3nm", "c3w4"):
                pats = ((1, 4), (2, 4), (2, 8), (4, 8)) if k == "c3nm" else ((2, 4), (2, 8), (4, 8))
                for i, (n, m) in enumerate(pats):
                    print("bench: workload %s, %d:%d ..." % (k, n, m), file=sys.stderr, flush=True)
                    table["%s_%d:%d" % (k, n, m)] = bench_workload(k, args.workload_iters or 200,
                                                                   dense_cmp=i == 0, nm=(n, m))
                    print("bench: workload %s, %d:%d, packed decode layout ..." % (k, n, m), file=sys.stderr,
                          flush=True)
                    table["%s_%d:%d_packed" % (k, n, m)] = bench_workload(k, args.workload_iters or 200,
                                                                          dense_cmp=False, nm=(n, m), packed=True)
                continue
            print("bench: workload %s ..." % k, file=sys.stderr, flush=True)
            it = args.workload_iters or (200 if W.WORKLOADS[k].klass != "large_n" else 20)
            if k != key:                                 # the headline's row-major product is timed above
                table[k] = bench_workload(k, it)
            if W.WORKLOADS[k].klass == "large_n" and k not in ("c1", key):
                print("bench: workload %s, packed prefill layout ..." % k, file=sys.stderr, flush=True)
                table[k + "_prefill"] = bench_workload(k, it, dense_cmp=False, prefill=True)
                print("bench: workload %s, packed prefill layout, activation-major B ..." % k, file=sys.stderr,
                      flush=True)
                table[k + "_prefill_bt"] = bench_workload(k, it, dense_cmp=False, prefill=True, bt=True)
            if W.WORKLOADS[k].residual:
                print("bench: workload %s, delta-coded residual ..." % k, file=sys.stderr, flush=True)
                table[k + "_delta"] = bench_workload(k, it, delta=True, dense_cmp=False)
                print("bench: workload %s, packed decode layout ..." % k, file=sys.stderr, flush=True)
                table[k + "_packed"] = bench_workload(k, it, dense_cmp=False, packed=True)
                print("bench: workload %s, packed decode layout, delta-coded residual ..." % k, file=sys.stderr,
                      flush=True)
                table[k + "_delta_packed"] = bench_workload(k, it, delta=True, dense_cmp=False, packed=True)
                print("bench: workload %s, packed decode layout, complement-bitmap residual ..." % k,
                      file=sys.stderr, flush=True)
                table[k + "_cbm_packed"] = bench_workload(k, it, dense_cmp=False, packed=True, cbm=True)
                print("bench: workload %s, packed decode layout, complement-bitmap residual, activation-major B ..."
                      % k, file=sys.stderr, flush=True)
                table[k + "_cbm_packed_bt"] = bench_workload(k, it, dense_cmp=False, packed=True, cbm=True, bt=True)
            elif W.WORKLOADS[k].klass == "small_n" and W.WORKLOADS[k].N == 16:
                print("bench: workload %s, packed decode layout ..." % k, file=sys.stderr, flush=True)
                table[k + "_packed"] = bench_workload(k, it, dense_cmp=False, packed=True)
                print("bench: workload %s, packed decode layout, activation-major B ..." % k, file=sys.stderr,
                      flush=True)
                table[k + "_packed_bt"] = bench_workload(k, it, dense_cmp=False, packed=True, bt=True)
        out["workloads"] = table
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
