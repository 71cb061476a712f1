"""Benchmark: paged attention steps on one MI355X.

Default workload (the one the headline metric is quoted on): GQA decode,
256 sequences, 32 query / 8 KV heads, head_dim 128, 16-token blocks, fp16
KV pool sized to the blocks needed plus 10% with a seeded permutation of
block ids, KV lengths U[1, 4096] (seed 47003), one new token per sequence.
``--workload N`` times one of the other synthetic workloads instead (1 tiny
MHA decode, 2 GPT-2-shaped batch: a decode step after the prefill, 4 shared
prefix + beam copy-on-write, 5 packed int8 chunked prefill + decode).

One step = the whole hot path over one batch with its inputs already in HBM:
``pa_copy_blocks`` (copy-on-write pairs, if any), ``pa_write_kv`` of the
step's new K/V rows through the slot mapping, then ``pa_attend`` (plan
kernel, split-K vector attention kernel and its log-sum-exp reduce, MFMA
attention kernel).  W warmup steps, then K timed steps between two
synchronisations (the headline value); then the same K steps again, each
recording fence-free HIP events on the library's stream right around the
attention kernels, which give the per-kernel durations of the roofline (the
events themselves cost a few microseconds of stream time, so they stay out
of the headline region).

Printed: one JSON line.  ``value`` is the KV-read throughput of the step in
GB/s: algorithmic bytes = sum over sequences of kv_len * kv_heads *
head_dim * 2 (K and V) * element bytes (+ one fp16 scale per (block, head)
per pool for int8) over the step time.
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

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_F16_TFLOPS = 2500.0
PMC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_gqa-decode-256_pmc.json")

WORKLOADS = {
    1: "tiny-mha-decode: 4 seqs (kv_len 40/20/16/30), 12/12 heads, head_dim 64, 8-block fp16 pool",
    2: "gpt2-batch decode step: 32 seqs after prefill of U[32,512] prompts, 12/12 heads, head_dim 64, fp16",
    3: "gqa-decode: 256 seqs, kv_len U[1,4096] (seed 47003), 32 q / 8 kv heads, head_dim 128, block 16, "
       "fp16 KV, 1 new token per seq (write + attend)",
    4: "prefix-share-beam-cow: 112 seqs over a shared 1024-token prefix, 16 requests x 4 beams, "
       "copy-on-write + write + attend, 32/8 heads, head_dim 128, fp16",
    5: "packed-int8: 8 chunks x 512 rows (context U[0,8192]) + 192 decode seqs (kv_len U[1,32768]), "
       "32/8 heads, head_dim 128, int8 KV with per-block-per-head fp16 scales",
    6: "gpt2-churn: 256 requests (prompts U[32,512], 64 new tokens each) through the continuous-batching "
       "scheduler over a 1152-block pool, <= 4096 rows and 64 sequences per step, 12/12 heads, head_dim 64",
}


class TimingEvents:
    """HIP events created with hipEventDisableSystemFence: recording them does
    not write back or invalidate caches, so they time the work between them
    without slowing it down (default events cost several microseconds each)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import ctypes
        self._ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def handle(self, i: int) -> int:
        return self.ev[i].value

    def record_all(self, stream: int) -> None:
        for e in self.ev:
            if self.hip.hipEventRecord(e, self._ct.c_void_p(stream)) != 0:
                raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = self._ct.c_float()
        if self.hip.hipEventElapsedTime(self._ct.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


class SideStream:
    """A second stream (default priority) and two untimed events for
    pa_attend's side-stream option: the row tiles of a packed batch run there,
    beside the decode units."""
    DISABLE_TIMING = 0x2

    def __init__(self):
        import ctypes
        import torch
        self.stream = torch.cuda.Stream()
        hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(2):
            e = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.DISABLE_TIMING)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def handles(self):
        return (self.stream.cuda_stream, self.ev[0].value, self.ev[1].value)


# the sources of the vector-path kernel whose HBM traffic the PMC summary records
DECODE_SOURCES = ("decode.hip", "pa_internal.h", "units.h")


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_47_amd", "csrc")
    for f in DECODE_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch of the default workload's attention kernel from
    the committed rocprofv3 PMC summary, or None when it is missing or was
    taken on other kernel sources."""
    try:
        with open(PMC_FILE) as f:
            p = json.load(f)
    except (OSError, ValueError):
        return None
    if p.get("source_hash") != source_hash():
        return None
    return p.get("hbm_bytes_per_launch")


def window_lo(pos: int, window: int) -> int:
    """First key a query at ``pos`` sees (0 without a sliding window)."""
    return max(0, pos - window + 1) if window > 0 else 0


def work_split(w, L, Q):
    """Algorithmic work of one step: (vector-path KV bytes, MFMA-path flops,
    total KV bytes).  Sequences with q_len * group >= 16 rows go to the row
    tiles (with groups of 16 or 32: from two query rows; single query rows
    then take the decode units on the matrix cores, which like the vector
    path are bound by KV bytes).  A decode-unit row reads the K and V of the
    keys it sees (int8: plus one
    scale per block and head for each); a sequence's total counts the keys
    any of its rows sees once; with a sliding window only keys inside it."""
    eb = 1 if w.kv_dtype == "i8" else 2
    bs = w.block_size
    per_tok = w.num_kv_heads * w.head_dim * 2 * eb
    per_blk = w.num_kv_heads * 2 * 2 if w.kv_dtype == "i8" else 0

    def keys_bytes(lo, hi):       # keys lo .. hi-1
        return (hi - lo) * per_tok + (-(-hi // bs) - lo // bs) * per_blk if hi > lo else 0

    vec_bytes, mfma_flops, total = 0, 0, 0
    for l, q in zip(L.tolist(), Q.tolist()):
        total += keys_bytes(window_lo(l - q, w.window), l)
        if q == 0:
            continue
        if q * w.group >= (2 * w.group if w.group >= 16 else 16):
            vis = sum(l - q + t + 1 - window_lo(l - q + t, w.window) for t in range(q))
            mfma_flops += 4 * w.head_dim * w.num_q_heads * vis
        else:
            vec_bytes += sum(keys_bytes(window_lo(l - q + t, w.window), l - q + t + 1) for t in range(q))
    return vec_bytes, mfma_flops, total


def _blas_name() -> str:
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')}"
    except Exception:   # older numpy: no dict form
        return "unknown"


def unique_kv_bytes(w, tables, L, Q) -> int:
    """KV bytes of the distinct physical blocks a step reads (a block shared
    by several sequences counts once, with its largest valid-token count)."""
    eb = 1 if w.kv_dtype == "i8" else 2
    valid = {}
    for row, n, q in zip(tables, L.tolist(), Q.tolist()):
        for j in range(window_lo(n - q, w.window) // w.block_size, -(-n // w.block_size)):
            b = int(row[j])
            valid[b] = max(valid.get(b, 0), min(w.block_size, n - j * w.block_size))
    return sum(valid.values()) * w.num_kv_heads * w.head_dim * 2 * eb


def hbm_ceilings(pool_bytes: int = 4 << 30, reps: int = 5, rounds: int = 3) -> dict:
    """What HBM delivers to plain reads on this GPU (pa_ceiling.h): a 4 GiB
    buffer read front to back (the best of four grid sizes), and the same
    buffer as two pools of 4 KiB K and V tiles read in a seeded random
    order, 16 or 64 pairs per wave with one or two more in flight (the
    decode kernel's access pattern at 256- and 1024-token partitions), the
    best of each.  Best of ``rounds`` timings of ``reps`` launches each, from
    events on the launching stream."""
    import torch
    from paged_kv_cache_47_amd import pa

    buf = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    half = pool_bytes // 2
    k_tiles, v_tiles = buf[:half], buf[half:]
    g = torch.Generator(device="cpu")
    g.manual_seed(47)
    ids = torch.randperm(half // 4096, generator=g).to(torch.int32).cuda()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_gbs(launch, nbytes):
        for _ in range(2):
            launch()
        best = 0.0
        for _ in range(rounds):
            a.record()
            for _ in range(reps):
                launch()
            b.record()
            b.synchronize()
            best = max(best, nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9)
        return best

    stream = {wg: best_gbs(lambda wg=wg: pa.pa_ceiling_stream_read(buf, sink, workgroups=wg), pool_bytes)
              for wg in (2048, 8192, 32768, 65536)}
    gather = {(n, d): best_gbs(lambda n=n, d=d: pa.pa_ceiling_gather(k_tiles, v_tiles, ids, sink, ids_per_wave=n,
                                                                     depth=d), pool_bytes)
              for n in (16, 64) for d in (1, 2)}
    del buf
    top, gtop = max(stream.values()), max(gather.values())
    return {"stream_read_gbs": round(top, 1), "stream_read_frac": round(top / PEAK_HBM_GBS, 4),
            "stream_read_by_workgroups": {str(k): round(v, 1) for k, v in stream.items()},
            "tile_gather_gbs": round(gtop, 1), "tile_gather_frac": round(gtop / PEAK_HBM_GBS, 4),
            "tile_gather_by_pairs_per_wave_and_depth": {f"{n}/{d}": round(v, 1) for (n, d), v in gather.items()},
            "note": "pa_ceiling_stream_read over 4 GiB (best grid); pa_ceiling_gather over 2 x 2 GiB of 4 KiB "
                    "K/V tiles in a seeded random order, 16 or 64 pairs per wave, 1 or 2 more in flight (best); "
                    "best of 3 x 5 launches each"}


def cpu_baseline(w, step: int, budget_s: float):
    """The oracle (gather through the block table + fp64 attention) on the
    first sequences of the same step, until ``budget_s`` of CPU time."""
    import oracle.attention as oatt
    import oracle.paging as opg
    st = opg.build_state(w)
    for s in range(step + 1):
        opg.apply_step(st, w.step(s).q_lens, w.window)
    sd = w.step(step)
    q_all = w.layer_acts(step, 0)[2]                 # layer 0 of a multi-layer pool
    K, V = w.pool_k, w.pool_v
    KS, VS = w.pool_k_scale, w.pool_v_scale
    if w.num_layers > 1:
        K, V = K[:, 0], V[:, 0]
        KS, VS = (None, None) if KS is None else (KS[:, 0], VS[:, 0])
    bs = w.block_size
    eb = 1 if w.kv_dtype == "i8" else 2
    starts = np.concatenate([[0], np.cumsum(sd.q_lens)[:-1]])
    t0 = time.perf_counter()
    done, kv_bytes = 0, 0
    for i in range(len(st.tables)):
        L, Q = st.lens[i], int(sd.q_lens[i])
        lo = oatt.window_start(L, Q, w.window)
        Kc = oatt.gather(K, st.tables[i], L, bs, KS, lo)
        Vc = oatt.gather(V, st.tables[i], L, bs, VS, lo)
        if Q:
            oatt.attend(q_all[starts[i]:starts[i] + Q], oatt.query_positions(L, Q), Kc, Vc, w.scale,
                        w.window, lo)
        done += 1
        kv_bytes += (L - lo) * w.num_kv_heads * w.head_dim * 2 * eb
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle", "blas": _blas_name(),
        "sample": f"first {done} of {len(st.tables)} sequences ({kv_bytes / 1e6:.1f} MB of KV), attention only "
                  f"(numpy fp64, BLAS threads={os.environ.get('OMP_NUM_THREADS', 'default')}), {dt:.1f} s"
                  + (" (on the pool as drawn: the int8 context replay is not part of the timed oracle work)"
                     if w.kv_dtype == "i8" else "")
                  + (" (layer 0 of the multi-layer pool)" if w.num_layers > 1 else ""),
        "seq_steps_per_s": round(done / dt, 3),
    }


# ------------------------------------------------------------ profile summaries ----
# Run on the host after the profiler runs (no GPU needed); they read the
# rocprofv3 CSV files and write the summaries kept under profiles/.

def _step_lengths(w, s: int = 0):
    """Post-write kv lengths and query rows of step ``s`` (host bookkeeping only)."""
    from paged_kv_cache_47_amd.workload import build_manager
    mgr, ids = build_manager(w)
    for i in range(s + 1):
        b = mgr.step(ids, w.step(i).q_lens)
    return b.seq_lens.astype(np.int64), b.q_lens.astype(np.int64)


def _read_counters(path: str):
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.setdefault((int(r["Dispatch_Id"]), r["Kernel_Name"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    return rows


def summarize_pmc(fetch_csv: str, write_csv: str, copy_mib: int, kernel_prefix: str, out: str, cmds) -> dict:
    """HBM bytes per launch of the decode kernel from one FETCH_SIZE run and
    one WRITE_SIZE run, each scaled by what the same counter reads for the
    plain device copy of ``copy_mib`` MiB that bench.py makes at the end of
    those runs (--copy-calibration-mib)."""
    copy_bytes = copy_mib << 20
    res = {"kernel_prefix": kernel_prefix, "commands": list(cmds)}
    per = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _read_counters(path)
        copies = [c[name] for (d, k), c in rows.items() if k.startswith("__amd_rocclr_copyBuffer") and name in c]
        calib = max(copies)                                     # KiB read (or written) for the big copy
        vals = [c[name] for (d, k), c in rows.items() if k.startswith(kernel_prefix) and name in c]
        per[name] = {"launches": len(vals), "KiB_per_launch": float(np.mean(vals)), "copy_KiB": calib,
                     "scale": copy_bytes / (calib * 1024.0)}
    fetch = per["FETCH_SIZE"]["KiB_per_launch"] * 1024 * per["FETCH_SIZE"]["scale"]
    write = per["WRITE_SIZE"]["KiB_per_launch"] * 1024 * per["WRITE_SIZE"]["scale"]
    import synthetic
    w = synthetic.CONFIGS[3]()
    L, Q = _step_lengths(w, 0)
    alg = work_split(w, L, Q)[0]
    res.update({"copy_bytes": copy_bytes, "counters": per,
                "hbm_bytes_per_launch": int(round(fetch + write)),
                "algorithmic_bytes_per_launch": int(alg),
                "traffic_over_algorithmic": round((fetch + write) / alg, 4),
                "source_hash": source_hash(), "source_files": list(DECODE_SOURCES)})
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    return res


def summarize_counters(csv_path: str, out: str, cmd: str, title: str, prefixes) -> None:
    """Per-dispatch averages of the SQ/GRBM counters of one rocprofv3 --pmc
    run for the kernels named by ``prefixes``, with the derived shares: MFMA
    busy and VALU issue per SIMD (1024 SIMDs, 32 shader engines, 8 XCDs on
    this part; per-SE counters are summed over the SEs, per-SIMD ones over the
    SIMDs, GRBM_GUI_ACTIVE over the XCDs)."""
    rows = _read_counters(csv_path)
    lines = [f"# {title}", "", "Command (repository root, one MI355X):", "", f"    {cmd}", ""]
    for pre in prefixes:
        per = {}
        n = 0
        for (d, k), c in rows.items():
            if k.startswith(pre):
                n += 1
                for name, v in c.items():
                    per[name] = per.get(name, 0.0) + v
        if not n:
            continue
        avg = {k: v / n for k, v in per.items()}
        lines += [f"## `{pre}` ({n} dispatches)", "", "| counter | per dispatch |", "|---|---|"]
        lines += [f"| {k} | {v:,.0f} |" for k, v in sorted(avg.items())]
        cyc = avg.get("GRBM_GUI_ACTIVE", 0) / 8 or avg.get("SQ_BUSY_CYCLES", 0) / 32
        if cyc:
            lines.append("")
            lines.append(f"Kernel cycles (GRBM_GUI_ACTIVE / 8 XCDs): {cyc:,.0f}.")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                lines.append(f"MFMA busy: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / cyc:.1%} of SIMD cycles.")
            if "SQ_ACTIVE_INST_VALU" in avg:
                lines.append(f"VALU issue: {avg['SQ_ACTIVE_INST_VALU'] * 4 / 1024 / cyc:.1%} of SIMD cycles "
                             "(quad-cycle units).")
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg and avg.get("SQ_VALU_MFMA_BUSY_CYCLES"):
                lines.append(f"VALU issued while the MFMA unit was busy: "
                             f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:.1%} of MFMA-busy cycles.")
            if "SQ_INSTS_VALU" in avg and "SQ_WAVES" in avg and avg["SQ_WAVES"]:
                lines.append(f"VALU instructions per wave: {avg['SQ_INSTS_VALU'] / avg['SQ_WAVES']:,.0f}; "
                             f"MFMA per wave: {avg.get('SQ_INSTS_MFMA', 0) / avg['SQ_WAVES']:,.0f}.")
        if avg.get("SQ_WAVE_CYCLES"):
            wc = avg["SQ_WAVE_CYCLES"]
            lines.append("")
            for name, what in (("SQ_ACTIVE_INST_ANY", "issuing an instruction"),
                               ("SQ_WAIT_ANY", "waiting on a counter or the barrier"),
                               ("SQ_WAIT_INST_ANY", "waiting for an issue slot"),
                               ("SQ_WAIT_INST_LDS", "with an LDS instruction waiting for issue")):
                if name in avg:
                    lines.append(f"Waves {what}: {avg[name] / wc:.1%} of wave cycles ({name} / SQ_WAVE_CYCLES).")
        lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_trace(stats_csv: str, out: str, cmd: str, title: str, alg_bytes: int = 0, alg_flops: int = 0,
                    kernel_prefix: str = "") -> None:
    """Kernel table from a rocprofv3 --kernel-trace --stats run, with the
    algorithmic rate of one kernel at its trace-average duration."""
    import csv
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    lines = [f"# {title}", "", "Command (repository root, one MI355X):", "", f"    {cmd}", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    avg = None
    for r in rows:
        name = r["Name"]
        lines.append(f"| `{name[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
        if kernel_prefix and name.startswith(kernel_prefix) and avg is None:
            avg = float(r["AverageNs"]) * 1e-9
    lines.append("")
    if avg and alg_bytes:
        lines.append(f"Algorithmic bytes per launch of `{kernel_prefix}`: {alg_bytes:,}; at the trace average "
                     f"({avg * 1e6:.1f} us) {alg_bytes / avg / 1e9:.0f} GB/s ({alg_bytes / avg / 1e9 / PEAK_HBM_GBS:.1%} "
                     f"of {PEAK_HBM_GBS:.0f} GB/s).")
    if avg and alg_flops:
        lines.append(f"Algorithmic flops per launch of `{kernel_prefix}`: {alg_flops:,}; at the trace average "
                     f"({avg * 1e6:.1f} us) {alg_flops / avg / 1e12:.1f} TFLOP/s "
                     f"({alg_flops / avg / 1e12 / PEAK_MFMA_F16_TFLOPS:.1%} of {PEAK_MFMA_F16_TFLOPS:.0f} TFLOP/s).")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _warm_clocks() -> None:
    """About 0.2 s of unrelated device work: set-up leaves the GPU idle long
    enough to drop its clocks."""
    import torch
    a_ = torch.randn(4096, 4096, device="cuda", dtype=torch.float16)
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.2:
        a_ = a_ @ a_
        a_ = a_ / a_.abs().amax()
        torch.cuda.synchronize()
    del a_
    torch.cuda.synchronize()


def end_to_end(args, w) -> dict:
    """Workload 2 run as a server would: the prefill step, then every decode
    step with its host bookkeeping (table growth, slot mapping), the copy of
    its metadata to the device, the KV writes and the attention of every
    layer.  Three ways to issue a decode step, each from a fresh pool:

    * eager: ``DeviceRun.prepare`` + ``run`` (the manager's step into numpy
      arrays, one packed metadata upload, the library calls marshalled anew);
    * prepared: ``StaticSteps`` (the native step straight into pinned memory,
      one copy to fixed device buffers, prepared library calls);
    * graph: the same, with the step's calls captured once in a HIP graph
      shaped for the largest length the run reaches, and replayed.

    Wall time over the decode steps (host included) and device time per step
    (events around each step's device work)."""
    import torch
    from paged_kv_cache_47_amd.workload import DeviceRun, StaticSteps
    out = {"layers": w.num_layers, "decode_steps": w.num_steps - 1}
    for mode in ("eager", "prepared", "graph"):
        run = DeviceRun(w)
        acts = [run.activations(s) for s in range(w.num_steps)]   # the model's outputs, already on the device
        x = run.prepare(0, acts=acts[0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run.run(x)
        e1.record()
        torch.cuda.synchronize()
        prefill_ms = e0.elapsed_time(e1)
        width = -(-(int(x.batch.seq_lens.max()) + w.num_steps - 1) // w.block_size)
        st = None
        if mode != "eager":
            st = StaticSteps(run, width)
            if mode == "graph":
                st.capture()
        _warm_clocks()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(w.num_steps)]
        for a_, b_ in ev:
            a_.record()
            b_.record()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(1, w.num_steps):
            if mode == "eager":
                x = run.prepare(s, acts=acts[s])
                ev[s][0].record()
                run.run(x)
            else:
                st.set_activations(acts=acts[s])
                st.host_step(exact_lengths=mode == "prepared")
                ev[s][0].record()
                st.launch() if mode == "prepared" else st.replay()
            ev[s][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        dev = [a_.elapsed_time(b_) for a_, b_ in ev[1:]]
        seqs = len(run.ids)
        dec = w.num_steps - 1
        out[mode] = {"seq_steps_per_s_wall": round(seqs * dec / wall, 1),
                     "seq_steps_per_s_device": round(seqs * dec / (sum(dev) * 1e-3), 1),
                     "wall_ms_per_step": round(wall / dec * 1e3, 4),
                     "device_ms_per_step": round(float(np.mean(dev)), 5)}
        if mode == "eager":
            out["prefill_ms"] = round(prefill_ms, 5)
        del st, run, acts, x
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    out["seq_steps"] = len(w.ctx_lens) * (w.num_steps - 1)
    out["note"] = ("a seq-step is one new token of one sequence through the KV write and attention of every "
                   "layer; wall: host bookkeeping + metadata copy + device work of every decode step, with the new "
                   "K/V and queries already on the device (copied into the fixed buffers in the prepared and "
                   "graph modes); device: events around each step's device work")
    return out


def serve_bench(args) -> dict:
    """Workload 6: the whole request stream through the native scheduler and
    the library, every step's bookkeeping, metadata copy, writes and
    attention in the timed region (the activations a model would produce are
    slices of buffers already on the device).  One untimed pass first."""
    import torch
    import synthetic
    from paged_kv_cache_47_amd.workload import ServeRun
    rs = synthetic.config6(num_layers=args.layers, kv_dtype=args.kv_dtype, system_prompts=args.system_prompts)
    dt = torch.bfloat16 if rs.kv_dtype == "bf16" else torch.float16
    lead = () if rs.num_layers == 1 else (rs.num_layers,)
    g = torch.Generator(device="cuda").manual_seed(rs.seed)
    big = [torch.randn((*lead, rs.max_batch_tokens, h, rs.head_dim), generator=g, device="cuda").to(dt)
           for h in (rs.num_kv_heads, rs.num_kv_heads, rs.num_q_heads)]

    def acts(step, rows):
        return tuple(b[..., :rows, :, :] if rs.num_layers == 1 else b[:, :rows] for b in big)

    def one_pass(timed):
        run = ServeRun(rs, acts=acts)
        ev, rows, prefill_rows = [], 0, 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while not run.done():
            if timed:
                a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a_.record()
            st, _ = run.step()
            if timed:
                b_.record()
                ev.append((a_, b_))
            rows += int(st.q_lens.sum())
            prefill_rows += int(st.q_lens[st.q_lens > 1].sum())
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return run, wall, ev, rows, prefill_rows

    one_pass(False)
    _warm_clocks()
    run, wall, ev, rows, prefill_rows = one_pass(True)
    steps = len(ev)
    dev_ms = sum(a_.elapsed_time(b_) for a_, b_ in ev)
    gen = run.sched.counts()["generated"]
    return {
        "metric": "continuous batching under churn: generated tokens (seq-steps) per second",
        "value": round(gen / wall, 1), "unit": "seq-steps/s", "n_gpus": 1, "steps": steps, "warmup": 1,
        "ms_per_step": round(wall / steps * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": rs.kv_dtype, "data": "synthetic",
        "config": {"workload": WORKLOADS[6] + (f" [{rs.num_layers} layers per block]" if rs.num_layers > 1 else "")
                   + (f" [prompts = one of {args.system_prompts} shared system prompts of U[64,256] tokens + "
                      "U[32,512] own tokens, through the prefix cache]" if args.system_prompts else ""),
                   "requests": int(len(rs.prompts)), "new_tokens": int(rs.new_tokens[0]),
                   "num_blocks": rs.num_blocks, "max_batch_tokens": rs.max_batch_tokens, "max_seqs": rs.max_seqs,
                   "lookahead": rs.lookahead, "max_skips": rs.max_skips, "layers": rs.num_layers},
        "generated_tokens": int(gen), "rows": rows, "prefill_rows": prefill_rows,
        "prompt_tokens": int(rs.prompts.sum()), "prompt_tokens_from_cache": int(run.sched.cached_tokens),
        "wall_s": round(wall, 4), "device_ms_per_step": round(dev_ms / steps, 5),
        "seq_steps_per_s_device": round(gen / (dev_ms * 1e-3), 1),
        "roofline": None,
        "note": "wall: the whole stream, host scheduling + metadata copy + writes + attention of every step; "
                "device: events around each step's work; no roofline line: the steps mix prefill (MFMA) and "
                "decode (vector) kernels of varying size (workloads 2, 3 and 5 rate each kernel)",
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the HBM read ceilings (stream read, random 4 KiB tile gather) in the JSON line")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--fused-write", action="store_true",
                    help="issue each layer's write and attention as one pa_write_attend call")
    ap.add_argument("--mfma-split-steps", type=int, default=0,
                    help="split row tiles walking more 64-key steps than this (0: the library's choice, -1: never)")
    ap.add_argument("--cold", type=int, default=-1, choices=(-1, 0, 1),
                    help="also time steps after a 1 GiB scratch write that evicts the 256 MB MALL "
                         "(default: for working sets under 512 MB, workloads 1, 2 and 4)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding-window attention over this many keys (0: full causal attention)")
    ap.add_argument("--layers", type=int, default=1,
                    help="workload 2 only: layers per block (GPT-2 small has 12); a step writes and attends "
                         "every layer over one set of metadata")
    ap.add_argument("--kv-dtype", default="f16", choices=("f16", "bf16", "i8"),
                    help="workloads 2, 3 and 6: the pool type (bf16 pools take and return bf16 activations; "
                         "i8, workload 6 only: int8 codes with per-block-per-head fp16 scales, fp16 activations)")
    ap.add_argument("--system-prompts", type=int, default=0,
                    help="workload 6: requests start with one of this many shared system prompts, served from "
                         "the prefix cache")
    ap.add_argument("--side-stream", action="store_true",
                    help="packed batches (workload 5): the row-tile kernel on a second stream beside the decode "
                         "kernels (pa_attend's side-stream option)")
    ap.add_argument("--w3-q-heads", type=int, default=32, choices=(8, 16, 32, 64, 128, 256),
                    help="workload 3: query heads over the 8 KV heads (128 and 256: groups of 16 and 32, on the "
                         "matrix-core decode kernel)")
    ap.add_argument("--w5-pool", default="i8", choices=("i8", "f16", "bf16"),
                    help="workload 5: the pool type of the same packed batch (f16/bf16: N(0,1) contents in place)")
    ap.add_argument("--w5-q-heads", type=int, default=32, choices=(32, 64, 128),
                    help="workload 5: query heads over the 8 KV heads (64: groups of eight; 128: groups of 16, "
                         "the decode rows on the matrix cores)")
    ap.add_argument("--w5-chunks", type=int, default=8,
                    help="workload 5: number of 512-query prefill chunks")
    ap.add_argument("--w5-chunk-ctx", type=int, default=-1,
                    help="workload 5: cached context of every chunk (-1: drawn from U[0,8192])")
    ap.add_argument("--w5-chunks-only", action="store_true",
                    help="workload 5: the 8 prefill chunks alone (no decode sequences): the MFMA kernel by itself")
    ap.add_argument("--no-share", action="store_true",
                    help="workload 4 control: every sequence owns its own copy of the prefix (no sharing, no forks)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (profiler byte-counter scale)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                    help="write the HBM-traffic summary of the decode kernel from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) made with --copy-calibration-mib; no GPU is used")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "OUT_MD", "COMMAND"),
                    help="write a kernel-trace summary from a rocprofv3 --stats file; no GPU is used")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("PMC_CSV", "OUT_MD", "COMMAND"),
                    help="write per-dispatch SQ/GRBM counter averages of --summary-kernel (semicolon-separated "
                         "prefixes) from a rocprofv3 --pmc run; no GPU is used")
    ap.add_argument("--summary-kernel", default="void pa::decode_kernel<128, 4, 0,",
                    help="kernel-name prefix the summaries rate")
    ap.add_argument("--summary-title", default="")
    ap.add_argument("--pmc-commands", nargs="*", default=[])
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        r = summarize_pmc(*args.summarize_pmc[:2], args.copy_calibration_mib or 1024, args.summary_kernel,
                          args.summarize_pmc[2], args.pmc_commands)
        print(json.dumps({k: r[k] for k in ("hbm_bytes_per_launch", "algorithmic_bytes_per_launch",
                                             "traffic_over_algorithmic", "source_hash")}))
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.summarize_counters[2],
                           args.summary_title or "SQ counters", args.summary_kernel.split(";"))
        return 0
    if args.summarize_trace:
        import synthetic
        if args.workload == 5:
            w = synthetic.config5(kv_dtype=args.w5_pool, num_decode=0 if args.w5_chunks_only else 192,
                                  num_q_heads=args.w5_q_heads, num_chunks=args.w5_chunks,
                                  chunk_ctx=None if args.w5_chunk_ctx < 0 else args.w5_chunk_ctx)
        elif args.workload == 3:
            w = synthetic.config3(kv_dtype=args.kv_dtype, num_q_heads=args.w3_q_heads)
        else:
            w = synthetic.CONFIGS[args.workload]()
        w.window = args.window
        L, Q = _step_lengths(w, 1 if args.workload == 2 else 0)
        vb, mf, _ = work_split(w, L, Q)
        mfma = "prefill" in args.summary_kernel
        summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.summarize_trace[2],
                        args.summary_title or f"{args.summary_kernel}: kernel trace",
                        0 if mfma else vb, mf if mfma else 0, args.summary_kernel)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    if args.workload == 6:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps(serve_bench(args)), flush=True)
        return 0

    import torch
    import synthetic
    from paged_kv_cache_47_amd import pa
    from paged_kv_cache_47_amd.workload import DeviceRun

    torch.cuda.set_device(0)
    if args.layers != 1 and args.workload not in (2, 6):
        print("--layers applies to workloads 2 and 6 only", file=sys.stderr)
        return 2
    if args.kv_dtype != "f16" and args.workload not in (2, 3, 6):
        print("--kv-dtype applies to workloads 2, 3 and 6 only", file=sys.stderr)
        return 2
    if args.kv_dtype == "i8" and args.workload != 6:
        print("--kv-dtype i8 applies to workload 6 (workload 5 is the int8 kernel workload)", file=sys.stderr)
        return 2
    if (args.w5_pool != "i8" or args.w5_chunks_only or args.w5_q_heads != 32 or args.w5_chunks != 8
            or args.w5_chunk_ctx >= 0) and args.workload != 5:
        print("--w5-pool, --w5-q-heads, --w5-chunks, --w5-chunk-ctx and --w5-chunks-only apply to workload 5 only",
              file=sys.stderr)
        return 2
    if args.workload == 4 and args.no_share:
        w = synthetic.config4(share=False)
    elif args.workload == 5:
        w = synthetic.config5(kv_dtype=args.w5_pool, num_decode=0 if args.w5_chunks_only else 192,
                              num_q_heads=args.w5_q_heads, num_chunks=args.w5_chunks,
                              chunk_ctx=None if args.w5_chunk_ctx < 0 else args.w5_chunk_ctx)
    elif args.workload == 2:
        w = synthetic.config2(num_layers=args.layers, kv_dtype=args.kv_dtype)
    elif args.workload == 3:
        w = synthetic.config3(kv_dtype=args.kv_dtype, num_q_heads=args.w3_q_heads)
    else:
        w = synthetic.CONFIGS[args.workload]()
    w.window = args.window
    run = DeviceRun(w)
    step_index = 0
    if args.workload == 2:            # prefill (step 0) first; the timed step is the first decode step
        x0 = run.prepare(0)
        run.run(x0)
        step_index = 1
    x = run.prepare(step_index)
    S = len(run.ids)
    L = x.batch.seq_lens.astype(np.int64)
    Q = x.batch.q_lens.astype(np.int64)
    vec_bytes, mfma_flops, kv_bytes = work_split(w, L, Q)
    kv_bytes *= w.num_layers                     # the step attends every layer
    need = pa.pa_attend_workspace_bytes(run.k_cache, w.num_q_heads, x.batch.seq_lens, x.batch.q_lens,
                                        partition_tokens=args.partition_tokens, window=w.window,
                                        mfma_split_steps=args.mfma_split_steps)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    n = args.warmup + args.steps
    evs = TimingEvents(4 * n)
    evs.record_all(torch.cuda.current_stream().cuda_stream)   # first records are slow: do them untimed
    torch.cuda.synchronize()

    # every step's library calls, marshalled once before anything is timed: copies (if any), then per
    # layer the KV write and the attention (layers after the first reuse the first one's plan); the
    # timed variant records the kernel events around the first layer's attention kernels
    kc, vc, ks, vs = run.k_cache, run.v_cache, run.k_scale, run.v_scale
    outs = [torch.empty_like(run.layer_acts(x, l)[2]) for l in range(w.num_layers)]
    side = SideStream().handles() if args.side_stream else None

    def step_calls(i, timed_kernel):
        calls = [pa.prepare_copy_blocks(kc, vc, x.copy_pairs, ks, vs)] if x.copy_pairs.shape[0] else []
        for layer in range(w.num_layers):
            nk, nv, q = run.layer_acts(x, layer)
            ev = tuple(evs.handle(4 * i + j) for j in range(4)) if (timed_kernel and layer == 0) else None
            att = dict(out=outs[layer], workspace=ws, k_scale=ks, v_scale=vs, partition_tokens=args.partition_tokens,
                       events=ev, window=w.window, layer=layer, reuse_plan=layer > 0, side=side,
                       mfma_split_steps=args.mfma_split_steps)
            if args.fused_write:
                calls.append(pa.prepare_write_attend(nk, nv, x.slot_mapping, q, kc, vc, x.block_tables, x.seq_lens,
                                                     x.q_lens, x.batch.seq_lens, x.batch.q_lens, w.scale, **att))
                continue
            calls.append(pa.prepare_write_kv(nk, nv, x.slot_mapping, kc, vc, ks, vs, layer=layer))
            calls.append(pa.prepare_attend(q, kc, vc, x.block_tables, x.seq_lens, x.q_lens, x.batch.seq_lens,
                                           x.batch.q_lens, w.scale, **att))
        return calls

    prepared = {(i, tk): step_calls(i, tk) for i in range(n) for tk in (True, False)}

    def step(i, timed_kernel=True):
        for c in prepared[(i, timed_kernel)]:
            c()

    # the region's own events, created and recorded once before anything is timed
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    t1.record()
    torch.cuda.synchronize()

    def timed(steps, timed_kernel):
        torch.cuda.synchronize()
        t0.record()
        for i in steps:
            step(i, timed_kernel)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / len(steps)

    # The host-side set-up leaves the GPU idle for seconds; its clocks then need about 20 ms of this
    # memory-bound work to settle (measured: with 5 warmup steps the first 50 timed steps of workload 3
    # ran 7% slower than the same steps after 50 ms of them).  So the step itself is issued, untimed,
    # for 50 ms before the W warmup steps.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < 0.05:
        step(0, False)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    # the timed region (the headline value) issues the steps exactly as a caller would, with no
    # timing events inside; the same steps then run again with events recorded right around the
    # attention kernels, which give the per-kernel durations of the roofline
    ms = timed(range(args.warmup, n), False)
    ms_events = timed(range(args.warmup, n), True)
    e2e = end_to_end(args, w) if args.workload == 2 else None
    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    roof = []
    # with shared blocks (workload 4) the HBM-bound figure counts each distinct block once:
    # the other reads of a shared prefix are cache hits, not HBM traffic
    shared = args.workload == 4 and not args.no_share
    roof_bytes = unique_kv_bytes(w, x.batch.block_tables, L, Q) if shared else vec_bytes
    if vec_bytes:
        k_all = [evs.elapsed_ms(4 * i, 4 * i + 1) for i in range(args.warmup, n)]
        k_ms = float(np.mean(k_all))
        ach = roof_bytes / (k_ms * 1e-3) / 1e9
        roof.append({"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": traffic_from_profile() if (args.workload == 3 and args.w3_q_heads == 32
                                                           and args.kv_dtype == "f16" and not args.partition_tokens
                                                           and not args.window) else None,
                     "kernel": ("decode_mfma_kernel (split-K units on the matrix cores)"
                                if w.num_q_heads // w.num_kv_heads >= 16 else "decode_kernel (split-K vector path)"),
                     "kernel_ms": round(k_ms, 5),
                     "kernel_ms_median": round(float(np.median(k_all)), 5),
                     "algorithmic_bytes_per_launch": roof_bytes})
        if shared:
            roof[-1]["logical_bytes_per_launch"] = vec_bytes
            roof[-1]["logical_gbs"] = round(vec_bytes / (k_ms * 1e-3) / 1e9, 2)
    if mfma_flops:
        k_all = [evs.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(args.warmup, n)]
        k_ms = float(np.mean(k_all))
        ach = mfma_flops / (k_ms * 1e-3) / 1e12
        roof.append({"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_MFMA_F16_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_kernel (MFMA path, fp16 16x16x32)", "kernel_ms": round(k_ms, 5),
                     "kernel_ms_median": round(float(np.median(k_all)), 5),
                     "algorithmic_flops_per_launch": mfma_flops})
    roof.sort(key=lambda r: -r["kernel_ms"])       # the dominant kernel first
    # cold steps last: they re-record the per-step kernel events read above
    cold = None
    if args.cold == 1 or (args.cold == -1 and args.workload in (1, 2, 4)):
        # each step after a 1 GiB scratch write (more than the 256 MB MALL): the step's own
        # device time from events right around it, the kernels' from the library's events
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a_, b_ in ce:
            a_.record()
            b_.record()
        torch.cuda.synchronize()
        for j, i in enumerate(range(args.warmup, n)):
            scratch.fill_(j & 0xff)
            ce[j][0].record()
            step(i)
            ce[j][1].record()
        torch.cuda.synchronize()
        st_ms = [a_.elapsed_time(b_) for a_, b_ in ce]
        cold = {"ms_per_step_median": round(float(np.median(st_ms)), 5),
                "value_median": round(kv_bytes / (float(np.median(st_ms)) * 1e-3) / 1e9, 2),
                "note": "each step after a 1 GiB scratch write evicting the MALL; median over the timed steps"}
        if vec_bytes:
            kc = float(np.median([evs.elapsed_ms(4 * i, 4 * i + 1) for i in range(args.warmup, n)]))
            cold.update({"decode_kernel_ms_median": round(kc, 5),
                         "decode_kernel_gbs": round(vec_bytes / (kc * 1e-3) / 1e9, 2)})
        del scratch
    res = {
        "metric": "paged decode attn: achieved KV-read HBM GB/s (% of peak); seq-steps/s",
        "value": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload] + (" [control: every sequence owns its prefix copy]"
                                                          if args.workload == 4 and args.no_share else "")
                   + (f" [sliding window of {args.window} keys]" if args.window else "")
                   + (f" [{w.num_layers} layers per block: every step writes and attends each]"
                      if w.num_layers > 1 else "")
                   + (" [bf16 KV, queries and outputs]" if w.kv_dtype == "bf16" else "")
                   + (f" [{args.w3_q_heads} query heads]" if args.w3_q_heads != 32 else "")
                   + (f" [{args.w5_q_heads} query heads]" if args.w5_q_heads != 32 else "")
                   + (" [row tiles on a side stream]" if args.side_stream else "")
                   + (" [write and attention as one call]" if args.fused_write else "")
                   + (f" [{args.w5_pool} pool with N(0,1) contents]" if args.w5_pool != "i8" else "")
                   + (f" [{args.w5_chunks} chunks]" if args.w5_chunks != 8 else "")
                   + (f" [every chunk over {args.w5_chunk_ctx} cached keys]" if args.w5_chunk_ctx >= 0 else "")
                   + (" [the prefill chunks only]" if args.w5_chunks_only else ""),
                   "num_seqs": S, "kv_tokens": int(L.sum()),
                   "query_rows": int(Q.sum()), "num_blocks": w.num_blocks,
                   "partition_tokens": args.partition_tokens, "mfma_split_steps": args.mfma_split_steps,
                   "window": args.window, "layers": w.num_layers},
        "pct_of_peak": round(100 * kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "seq_steps_per_s": round(S / (ms * 1e-3), 1),
        "ms_per_step_with_kernel_events": round(ms_events, 5),
        "kv_bytes_per_step": kv_bytes,
        "roofline": roof[0] if roof else None,
    }
    if len(roof) > 1:
        res["roofline_other"] = roof[1:]
    if cold is not None:
        res["cold"] = cold
    if e2e is not None:
        res["end_to_end"] = e2e
    if args.workload == 4:
        ub = unique_kv_bytes(w, x.batch.block_tables, L, Q)
        res["unique_kv_bytes_per_step"] = ub
        res["value_unique"] = round(ub / (ms * 1e-3) / 1e9, 2)
        res["pct_of_peak"] = round(100 * ub / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)   # of unique bytes
        res["config"]["shared_prefix"] = not args.no_share
    if not args.no_ceilings:
        c = hbm_ceilings()
        if roof and roof[0]["bound"] == "hbm":
            c["roofline_over_tile_gather"] = round(roof[0]["achieved"] / c["tile_gather_gbs"], 4)
        res["hbm_ceilings"] = c
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, step_index, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
