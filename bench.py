"""Benchmark: paged GQA decode on one MI355X.

Workload (the one the headline metric is quoted on): 256 sequences, 32 query
/ 8 KV heads, head_dim 128, 16-token blocks, fp16 KV pool sized to the
blocks needed plus 10% with a seeded permutation of block ids, KV lengths
U[1, 4096] (seed 47003), one new token per sequence.

One step = the whole hot path over that batch with its metadata already in
HBM: ``pa_write_kv`` of the 256 new K/V rows through the slot mapping, then
``pa_attend`` (plan kernel, split-K vector attention kernel, log-sum-exp
reduce).  W warmup steps, then K timed steps between two synchronisations.

Printed (one JSON line): KV-read throughput of the step in GB/s (algorithmic
bytes: sum over sequences of kv_len * kv_heads * head_dim * 2 (K and V) * 2
bytes), seq-steps/s, the roofline of the dominant kernel (the split-K
attention kernel, timed with HIP events the library records around it on
the same stream) and the CPU oracle timed on a bounded sample.
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
DOMINANT = "decode_kernel"
PMC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_gqa-decode-256_pmc.json")


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

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = self._ct.c_float()
        if self.hip.hipEventElapsedTime(self._ct.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_47_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(n_launch_units: float):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None
    when it is missing or was taken on other kernel sources."""
    try:
        with open(PMC_FILE) as f:
            p = json.load(f)
    except (OSError, ValueError):
        return None
    if p.get("source_hash") != source_hash():
        return None
    return p.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s: float):
    """The oracle (gather through the block table + fp64 attention) on the
    first sequences of the same workload, until ``budget_s`` of CPU time."""
    import oracle.attention as oatt
    import oracle.paging as opg
    st = opg.build_state(w)
    slots, _ = opg.apply_step(st, w.step(0).q_lens)
    q = w.step(0).q
    K, V = w.pool_k, w.pool_v
    bs = w.block_size
    t0 = time.perf_counter()
    done, kv_bytes = 0, 0
    for i in range(len(st.tables)):
        L = st.lens[i]
        Kc = oatt.gather(K, st.tables[i], L, bs)
        Vc = oatt.gather(V, st.tables[i], L, bs)
        oatt.attend(q[i:i + 1], oatt.query_positions(L, 1), Kc, Vc, w.scale)
        done += 1
        kv_bytes += L * w.num_kv_heads * w.head_dim * 2 * 2
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {
        "value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"first {done} of {len(st.tables)} sequences ({kv_bytes / 1e6:.1f} MB of KV), "
                  f"attention only (numpy fp64, BLAS threads={os.environ.get('OMP_NUM_THREADS', 'default')}), "
                  f"{dt:.1f} s",
        "seq_steps_per_s": round(done / dt, 3),
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (profiler byte-counter scale)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import torch
    import synthetic
    from paged_kv_cache_47_amd import pa
    from paged_kv_cache_47_amd.workload import DeviceRun

    torch.cuda.set_device(0)
    w = synthetic.config3()
    run = DeviceRun(w)
    x = run.prepare(0)
    S = len(run.ids)
    L = x.batch.seq_lens.astype(np.int64)
    kv_bytes = int(L.sum()) * w.num_kv_heads * w.head_dim * 2 * 2
    out = torch.empty_like(x.q)
    need = pa.pa_attend_workspace_bytes(run.k_cache, w.num_q_heads, x.batch.seq_lens, x.batch.q_lens,
                                        partition_tokens=args.partition_tokens)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    n = args.warmup + args.steps
    evs = TimingEvents(2 * n)
    torch.cuda.synchronize()

    def step(i, timed_kernel=True):
        run.write(x)
        ev = (evs.handle(2 * i), evs.handle(2 * i + 1), None, None) if timed_kernel else None
        pa.pa_attend(x.q, run.k_cache, run.v_cache, x.block_tables, x.seq_lens, x.q_lens, x.batch.seq_lens,
                     x.batch.q_lens, w.scale, out=out, workspace=ws, partition_tokens=args.partition_tokens,
                     events=ev)

    def timed(steps, timed_kernel):
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in steps:
            step(i, timed_kernel)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / len(steps)

    for i in range(args.warmup):
        step(i)
    # the timed region: every step also records events around the attention kernel
    ms = timed(range(args.warmup, n), True)
    # the same steps without those events
    ms_plain = timed(range(args.warmup, n), False)
    if args.copy_calibration_mib:
        # a plain device copy of known size, for scaling rocprofv3 byte counters
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    k_ms = [evs.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.warmup, n)]
    k_avg = float(np.mean(k_ms))
    achieved = kv_bytes / (k_avg * 1e-3) / 1e9
    traffic = traffic_from_profile(1)
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
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "gqa-decode: 256 seqs, kv_len U[1,4096] (seed 47003), 32 q / 8 kv heads, "
                               "head_dim 128, block 16, fp16 KV, 1 new token per seq (write + attend)",
                   "num_seqs": S, "kv_tokens": int(L.sum()), "num_blocks": w.num_blocks,
                   "partition_tokens": args.partition_tokens},
        "pct_of_peak": round(100 * kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "seq_steps_per_s": round(S / (ms * 1e-3), 1),
        "ms_per_step_without_kernel_events": round(ms_plain, 5),
        "value_without_kernel_events": round(kv_bytes / (ms_plain * 1e-3) / 1e9, 2),
        "kv_bytes_per_step": kv_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": DOMINANT, "kernel_ms": round(k_avg, 5),
                     "algorithmic_bytes_per_launch": kv_bytes},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
