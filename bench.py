#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the hot path over one batch of seeded synthetic input: copy_blocks (copy on
write of diverging shared blocks), reshape_and_cache (the step's new K/V into their slots), decode,
prefill chunk -- each stage present in the workload. The default workload is the LLaMA-2-7B-shaped
single-layer decode: 64 sequences of U{512..4096} tokens, 32 query = 32 kv heads of 128, fp16,
16-token blocks from a seeded permutation of a pool sized to the needed blocks + 10%.

Prints ONE JSON line:
  value        algorithmic bytes of the whole step / time per step (GB/s), inputs resident in HBM;
  roofline     for the dominant kernel (decode): algorithmic bytes per launch / its average
               duration from HIP events recorded on the launch stream during the timed steps
               (timing-only events without the system-scope fence, see TimingEvents),
               against the 8 TB/s HBM peak; traffic = HBM bytes per launch from the workload's
               committed counter record (profiles/<workload>[_fp8]_traffic.json) when it was taken
               on the current decode sources, else null;
  roofline_prefill  (steps with a prefill chunk) the chunk's causal FLOPs / its event time against
               the 2.5 PFLOP/s dense bf16 MFMA peak, with the MFMA-busy share of SIMD cycles from
               the committed counter record of the current prefill sources, else null. Steps
               whose chunks are all short (drafted tokens, GpuStep.multi_token) read them with
               pa_decode_multi instead: its roofline is HBM, algorithmic bytes as for prefill; in
               a step with no one-token decodes it is also the line's roofline and cpu_baseline;
  step_tokens_per_s  query tokens the step attends for (decode sequences + prefill rows) / step
               time: the mixed step's 2048-token budget per step;
  cpu_baseline the CPU oracle (float64) timed on this host over the workload's decode (a bounded
               sample when it is long); cpu_baseline_prefill the oracle's prefill over a sample of
               chunk rows, in GFLOP/s.
  decode_ms, prefill_ms: mean of the per-call event times (their 10th/50th/90th percentiles
               beside them; decode_us_per_call the same mean in microseconds). Decode contexts are
               far larger than the 256 MB Infinity Cache, so each step reads them from HBM;
               --evict-mb 512 also displaces every cache level before each timed decode, to show
               that.
  stages       copy_blocks and reshape_and_cache (where the step has them), each timed alone after
               the steps: mean event time per call, algorithmic bytes (below) and their rate
               against the 8 TB/s HBM peak;
  graph        (--graph) the same step recorded once as a HIP graph and replayed: time per step
               and the rates above over it, for steps whose kernels are short enough that host
               launches show.

Algorithmic bytes (what the method must move, per stage; E = 2 bytes per cache element, 1 with
--kv-cache fp8, whose caches hold E4M3 codes):
  decode   sum_s L_s * 2 * H_kv * D * E (each valid token's K and V row once) + query + output;
           with shared-prefix groups read once, a group's common blocks count once for the group
           (the per-sequence count is reported as decode_logical_bytes);
  scatter  2 * T * H_kv * D * 2 read + 2 * T * H_kv * D * E written;
  copy     pairs * 2 caches * (16 * H_kv * D * E) read + the same written;
  prefill  K/V rows of the context once + query + output (its roofline is MFMA: 4*D*H_q*sum(p+1)).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "paged_kv_cache_99_amd", "csrc")
# sources of the decode kernels and of the prefill kernel: a committed counter record quotes the
# hash of the sources it was taken on, and is used only while that hash matches
DECODE_SRCS = [os.path.join(CSRC, f) for f in ("decode.hip", "pa_device.h", "pa_internal.h")]
PREFILL_SRCS = [os.path.join(CSRC, f) for f in ("prefill.hip", "pa_device.h", "pa_internal.h")]
PROFILES = os.path.join(ROOT, "profiles")


def decode_bytes(w, esize=2):
    nd = w.n_decode
    kv = int(np.sum(w.seq_lens[:nd].astype(np.int64))) * 2 * w.H_kv * w.D * esize
    return kv + 2 * nd * w.H_q * w.D * 2


def decode_unique_bytes(w, esize=2):
    """Bytes when every group's common blocks are read once (shared-prefix workloads); esize:
    bytes per cached K/V element (2, or 1 for E4M3 caches)."""
    meta = getattr(w, "meta", {}) or {}
    if "group_starts" not in meta:
        return decode_bytes(w, esize)
    nd = w.n_decode
    gs = np.asarray(meta["group_starts"])
    pre = np.asarray(meta["shared_prefix"], np.int64)[:nd]
    lens = w.seq_lens[:nd].astype(np.int64)
    shared = int(sum(pre[gs[g]] for g in range(len(gs) - 1) if gs[g + 1] > gs[g]))
    tokens = shared + int(np.sum(lens - pre))
    return tokens * 2 * w.H_kv * w.D * esize + 2 * nd * w.H_q * w.D * 2


def scatter_bytes(w, esize=2):
    return 2 * len(w.slot_mapping) * w.H_kv * w.D * (2 + esize)


def copy_bytes(w, esize=2):
    return 4 * len(w.copy_pairs) * 16 * w.H_kv * w.D * esize


def prefill_bytes_flops(w, esize=2):
    nd = w.n_decode
    lens = w.seq_lens[nd:].astype(np.int64)
    cu = np.asarray(w.cu_q_lens, np.int64)
    qlen = np.diff(cu)
    kv = int(np.sum(lens)) * 2 * w.H_kv * w.D * esize
    rows = int(cu[-1]) if len(cu) else 0
    flops = 0
    for L, ql in zip(lens, qlen):
        first = L - ql                       # position of the chunk's first row
        flops += 4 * w.D * w.H_q * int(np.sum(np.arange(first, L) + 1))
    return kv + 2 * rows * w.H_q * w.D * 2, flops


def src_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def record_tag(workload, fp8, shared_prefix_read_once):
    """Name of a workload's counter records under profiles/: <workload>[_fp8][_per_sequence]."""
    meta_shared = workload.startswith("prefix_sharing")
    return workload + ("_fp8" if fp8 else "") + \
        ("_per_sequence" if meta_shared and not shared_prefix_read_once else "")


def committed_record(tag, kind, srcs):
    """profiles/<tag>_<kind>.json when its recorded source hash matches the current sources."""
    try:
        with open(os.path.join(PROFILES, f"{tag}_{kind}.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("src_sha256_16") == src_hash(srcs) else None


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, max_seconds, fp8=None):
    """Time the float64 oracle over the workload's decode (a bounded sample when it is long), on
    every host thread, then on one thread over a sample of a quarter of that time.
    fp8 = (k_scale, v_scale): the oracle's E4M3 decode over its own quantization of the pool."""
    import oracle
    nd = w.n_decode
    threads = oracle.max_threads()
    esize = 2
    if fp8 is not None:
        esize = 1
        k8 = oracle.quantize_e4m3(w.k_cache, w.dtype, fp8[0])
        v8 = oracle.quantize_e4m3(w.v_cache, w.dtype, fp8[1])

    def timed(nthreads, seconds, step):
        # grow the sample by whole sequences until the next batch would pass `seconds`
        done_tokens, elapsed, n_seq = 0, 0.0, 0
        t0 = time.perf_counter()
        while n_seq < nd:
            take = np.arange(n_seq, min(nd, n_seq + step))
            pairs = np.array([(s, h) for s in take for h in range(w.H_q)], np.int32)
            if fp8 is None:
                oracle.decode(w.query_decode, w.k_cache, w.v_cache, w.block_tables[:nd],
                              w.seq_lens[:nd], w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype,
                              w.scale, pairs=pairs, nthreads=nthreads)
            else:
                oracle.decode_fp8(w.query_decode, k8, v8, w.block_tables[:nd], w.seq_lens[:nd],
                                  w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale, fp8[0],
                                  fp8[1], pairs=pairs, nthreads=nthreads)
            n_seq += len(take)
            done_tokens += int(np.sum(w.seq_lens[take]))
            elapsed = time.perf_counter() - t0
            if elapsed > seconds:
                break
        nbytes = done_tokens * 2 * w.H_kv * w.D * esize + 2 * n_seq * w.H_q * w.D * 2
        return n_seq, done_tokens, nbytes, elapsed

    n_seq, done_tokens, nbytes, elapsed = timed(threads, max_seconds, max(1, nd // 8))
    n1, _, b1, e1 = timed(1, max_seconds / 4, 1)
    what = "E4M3 decode" if fp8 is not None else "decode"
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"float64 oracle {what} of {n_seq} of {nd} sequences x {w.H_q} query heads "
                      f"({done_tokens} context tokens, {nbytes / 1e9:.3f} GB of K/V) in "
                      f"{elapsed:.2f} s, pool before the step's scatter",
            "seconds": round(elapsed, 3),
            "cpu_model": cpu_model(),
            "single_thread": {"value": round(b1 / e1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"{n1} of {nd} sequences in {e1:.2f} s"}}


def cpu_baseline_multi(w, max_seconds, fp8=None):
    """The float64 oracle over the workload's short chunks (multi-token rows: every row and query
    head of each sampled sequence), sequences taken in order until the sample passes max_seconds,
    on every host thread; rate in GB/s of each sampled sequence's K/V read once (the algorithmic
    bytes of pa_decode_multi)."""
    import oracle
    nd = w.n_decode
    cu = np.asarray(w.cu_q_lens, np.int64)
    S = len(cu) - 1
    threads = oracle.max_threads()
    esize = 2
    if fp8 is not None:
        esize = 1
        k8 = oracle.quantize_e4m3(w.k_cache, w.dtype, fp8[0])
        v8 = oracle.quantize_e4m3(w.v_cache, w.dtype, fp8[1])
    lens = w.seq_lens[nd:].astype(np.int64)
    n_seq, elapsed, t0 = 0, 0.0, time.perf_counter()
    step = max(1, S // 8)
    while n_seq < S:
        take = np.arange(n_seq, min(S, n_seq + step))
        pairs = np.array([(r, h) for s in take for r in range(cu[s], cu[s + 1])
                          for h in range(w.H_q)], np.int32)
        if len(pairs):
            if fp8 is None:
                oracle.prefill(w.query_prefill, w.k_cache, w.v_cache, w.block_tables[nd:],
                               w.seq_lens[nd:], w.cu_q_lens, w.H_q, w.H_kv, w.D, w.num_blocks,
                               w.dtype, w.scale, rows=pairs, nthreads=threads)
            else:
                oracle.prefill_fp8(w.query_prefill, k8, v8, w.block_tables[nd:], w.seq_lens[nd:],
                                   w.cu_q_lens, w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype,
                                   w.scale, fp8[0], fp8[1], rows=pairs, nthreads=threads)
        n_seq += len(take)
        elapsed = time.perf_counter() - t0
        if elapsed > max_seconds:
            break
    rows = int(cu[n_seq] - cu[0])
    nbytes = int(np.sum(lens[:n_seq])) * 2 * w.H_kv * w.D * esize + 2 * rows * w.H_q * w.D * 2
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"float64 oracle of the multi-token rows of {n_seq} of {S} sequences "
                      f"({rows} rows x {w.H_q} query heads, {nbytes / 1e9:.3f} GB of K/V read "
                      f"once per sequence) in {elapsed:.2f} s, pool before the step's scatter",
            "seconds": round(elapsed, 3),
            "cpu_model": cpu_model()}


def cpu_baseline_prefill(w, max_seconds, fp8=None):
    """The float64 oracle's prefill of a sample of the workload's chunk rows (every query head of
    each sampled row), on every host thread, grown until it passes max_seconds; rate in GFLOP/s of
    the causal attention it computed (4 * D per visible key and (row, head))."""
    import oracle
    nd = w.n_decode
    cu = np.asarray(w.cu_q_lens, np.int64)
    total = int(cu[-1])
    threads = oracle.max_threads()
    lens = w.seq_lens[nd:].astype(np.int64)
    if fp8 is not None:
        k8 = oracle.quantize_e4m3(w.k_cache, w.dtype, fp8[0])
        v8 = oracle.quantize_e4m3(w.v_cache, w.dtype, fp8[1])

    def visible(r):  # keys row r attends
        s = int(np.searchsorted(cu, r, side="right") - 1)
        return int(lens[s] - (cu[s + 1] - cu[s]) + (r - cu[s]) + 1)

    n_rows, elapsed, flops = 8, 0.0, 0
    while True:
        rows = np.unique(np.linspace(0, total - 1, min(n_rows, total)).astype(np.int64))
        pairs = np.array([(r, h) for r in rows for h in range(w.H_q)], np.int32)
        t0 = time.perf_counter()
        if fp8 is None:
            oracle.prefill(w.query_prefill, w.k_cache, w.v_cache, w.block_tables[nd:],
                           w.seq_lens[nd:], w.cu_q_lens, w.H_q, w.H_kv, w.D, w.num_blocks,
                           w.dtype, w.scale, rows=pairs)
        else:
            oracle.prefill_fp8(w.query_prefill, k8, v8, w.block_tables[nd:], w.seq_lens[nd:],
                               w.cu_q_lens, w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale,
                               fp8[0], fp8[1], rows=pairs)
        elapsed = time.perf_counter() - t0
        flops = sum(4 * w.D * w.H_q * visible(int(r)) for r in rows)
        if elapsed > max_seconds / 4 or len(rows) >= total:
            break
        n_rows *= 2
    return {"value": round(flops / elapsed / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"float64 oracle prefill of {len(rows)} of {total} chunk rows (evenly "
                      f"spaced) x {w.H_q} query heads, {flops / 1e9:.2f} GFLOP of causal "
                      f"attention, in {elapsed:.2f} s, pool before the step's scatter",
            "seconds": round(elapsed, 3)}


class TimingEvents:
    """Pairs of HIP timing events created with hipEventDisableSystemFence (hip_runtime_api.h).

    Recording a default event adds a system-scope release and acquire: a cache writeback and
    invalidation between the measured kernels and the work around them, which costs several
    microseconds per event and slows what follows. These events only write timestamps. They come
    from the HIP runtime this process has already mapped (torch's, which the library shares).
    """
    DISABLE_SYSTEM_FENCE = 0x20000000

    @staticmethod
    def _loaded_hip_runtime():
        """Path of the libamdhip64 already mapped into this process (dlopen of the same file returns
        the loaded library), else its usual soname."""
        try:
            with open("/proc/self/maps") as f:
                for line in f:
                    path = line.split()[-1] if len(line.split()) >= 6 else ""
                    if os.path.basename(path).startswith("libamdhip64.so"):
                        return path
        except OSError:
            pass
        return "libamdhip64.so.7"

    def __init__(self, pairs):
        import ctypes
        self._ct = ctypes
        hip = ctypes.CDLL(self._loaded_hip_runtime())
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip = hip
        self._ev = []
        for _ in range(2 * pairs):
            e = ctypes.c_void_p()
            self._check(hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE),
                        "hipEventCreateWithFlags")
            self._ev.append(e)

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: hipError_t {rc}")

    def record(self, i, end, stream):
        """Record the start (end=False) or end event of pair i on a torch stream."""
        self._check(self._hip.hipEventRecord(self._ev[2 * i + int(end)], stream.cuda_stream),
                    "hipEventRecord")

    def elapsed_ms(self, i):
        """Milliseconds between the two events of pair i (both must have completed)."""
        ms = self._ct.c_float()
        self._check(self._hip.hipEventElapsedTime(self._ct.byref(ms), self._ev[2 * i],
                                                  self._ev[2 * i + 1]), "hipEventElapsedTime")
        return float(ms.value)

    def close(self):
        for e in self._ev:
            self._hip.hipEventDestroy(e)
        self._ev = []


def calibration_copy(g, pairs):
    """Copy `pairs` blocks src = 0..pairs-1 -> dst = pairs..2*pairs-1 in both caches (the timed steps
    are over; the pool contents no longer matter) and report the bytes a perfect copy moves."""
    import torch
    from paged_kv_cache_99_amd import binding
    nb = g.k_cache.shape[0]
    pairs = min(pairs, nb // 2)
    mapping = torch.stack([torch.arange(pairs), torch.arange(pairs, 2 * pairs)], 1)
    mapping = mapping.to(torch.int32).contiguous().to(g.device)
    torch.cuda.synchronize()
    binding.copy_blocks(g.k_cache, g.v_cache, mapping)
    torch.cuda.synchronize()
    per_cache = pairs * g.k_cache[0].numel() * g.k_cache.element_size()
    print(f"[bench] calibration copy: {pairs} blocks x 2 caches = {2 * per_cache} bytes read and "
          f"{2 * per_cache} bytes written", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama2_7b_decode")
    ap.add_argument("--partition", type=int, default=None, help="decode partition size override")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="decode shared-prefix groups per sequence instead of reading each "
                         "group's common blocks once")
    ap.add_argument("--kv-cache", choices=["auto", "fp8"], default="auto",
                    help="fp8: E4M3 caches (quantizing scatter, E4M3 decode and prefill)")
    ap.add_argument("--k-scale", type=float, default=0.03, help="E4M3 key scale")
    ap.add_argument("--v-scale", type=float, default=0.02, help="E4M3 value scale")
    ap.add_argument("--print-decode-src-hash", action="store_true",
                    help="print the hashes of the decode and of the prefill sources (recorded "
                         "with counter summaries)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="PAIRS",
                    help="after timing, copy PAIRS whole blocks with pa_copy_blocks (a plain copy of "
                         "known size, for scaling HBM byte counters)")
    ap.add_argument("--evict-mb", type=int, default=0, metavar="MB",
                    help="read an MB-megabyte buffer before each timed decode (outside the decode "
                         "events, inside the step time) so that no cache level holds K/V rows from "
                         "the previous step; 512 exceeds the 256 MB Infinity Cache twice over")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step recorded once as a HIP graph and replayed (reported "
                         "under \"graph\"; the line's value stays the eager step's)")
    args = ap.parse_args()
    if args.print_decode_src_hash:
        print(src_hash(DECODE_SRCS), src_hash(PREFILL_SRCS))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library does not shard the hot path across GPUs "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import pa_workloads as W
    from paged_kv_cache_99_amd.step import GpuStep

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    w = W.named(args.workload)
    print(f"[bench] workload {w.name}: {len(w.seq_lens)} sequences, pool {w.num_blocks} blocks, "
          f"built in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    fp8 = args.kv_cache == "fp8"
    esize = 1 if fp8 else 2
    g = GpuStep(w, partition_size=args.partition,
                shared_prefix=not args.no_shared_prefix,
                kv_cache=args.kv_cache, k_scale=args.k_scale, v_scale=args.v_scale)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        g.run()
    torch.cuda.synchronize()

    K = args.steps
    ev = TimingEvents(K)   # decode call of each step
    evp = TimingEvents(K)  # prefill call of each step
    has_prefill = g.pre_query.shape[0] > 0
    # eviction by reading: a write would leave dirty lines whose write-back competes with the
    # decode's reads
    evict = (torch.zeros(args.evict_mb << 18, dtype=torch.int32, device="cuda")
             if args.evict_mb > 0 else None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        g.copy()
        g.scatter()
        if evict is not None:
            torch.amax(evict)
        ev.record(i, False, stream)
        g.decode()
        ev.record(i, True, stream)
        if has_prefill:
            evp.record(i, False, stream)
            g.prefill()
            evp.record(i, True, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K
    dec_t = [ev.elapsed_ms(i) for i in range(K)] if g.n_decode else [0.0]
    pre_t = [evp.elapsed_ms(i) for i in range(K)] if has_prefill else [0.0]
    ev.close()
    evp.close()

    # the copy and scatter stages, each timed alone after the steps (K calls back to back, events
    # around each): markers around them inside the timed steps stalled some steps' launches by
    # hundreds of microseconds. Repeating a step's copies and slot writes leaves the pool as it is.
    stage_us = {}
    for name, fn, present in (("copy_blocks", g.copy, len(w.copy_pairs) > 0),
                              ("reshape_and_cache", g.scatter, len(w.slot_mapping) > 0)):
        if present:
            e = TimingEvents(K)
            for i in range(K):
                e.record(i, False, stream)
                fn()
                e.record(i, True, stream)
            torch.cuda.synchronize()
            stage_us[name] = float(np.mean([e.elapsed_ms(i) for i in range(K)])) * 1e3
            e.close()
    dec_ms = float(np.mean(dec_t))
    pre_ms = float(np.mean(pre_t))

    graph_ms = None
    if args.graph:
        graph = g.capture()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / K
        del graph

    if args.copy_calibration:
        calibration_copy(g, args.copy_calibration)

    d_bytes = decode_bytes(w, esize)
    u_bytes = decode_unique_bytes(w, esize) if g.shared_prefix else d_bytes
    p_bytes, p_flops = prefill_bytes_flops(w, esize)
    step_bytes = u_bytes + scatter_bytes(w, esize) + copy_bytes(w, esize) + p_bytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_gbs = u_bytes / (dec_ms * 1e-3) / 1e9 if dec_ms > 0 else 0.0
    tag = record_tag(w.name, fp8, g.shared_prefix)
    trec = committed_record(tag, "traffic", DECODE_SRCS) if g.n_decode else None
    traffic = trec.get("hbm_bytes_per_launch") if trec else None
    step_tokens = int(w.n_decode) + int(g.pre_query.shape[0])
    out = {
        "metric": "pa_decode HBM GB/s (% of 8 TB/s peak) + decode tokens/s, 7B-shaped layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "num_seqs": int(w.n_decode),
            "q_heads": w.H_q, "kv_heads": w.H_kv, "head_dim": w.D, "block_size": 16,
            "seq_lens": [int(w.seq_lens[:w.n_decode].min()), int(w.seq_lens[:w.n_decode].max())]
            if w.n_decode else None,
            "context_tokens": int(np.sum(w.seq_lens[:w.n_decode])),
            "pool_blocks": int(w.num_blocks),
            "partition_size": g.partition_size,
            "copy_pairs": int(len(w.copy_pairs)),
            "scatter_tokens": int(len(w.slot_mapping)),
            "prefill_rows": int(g.pre_query.shape[0]),
            "shared_prefix_read_once": bool(g.shared_prefix),
            "kv_cache_dtype": "fp8_e4m3" if fp8 else w.dtype,
            "evict_mb": args.evict_mb,
        },
        "decode_tokens_per_s": round(w.n_decode / (ms_per_step * 1e-3), 1),
        "step_tokens": step_tokens,
        "step_tokens_per_s": round(step_tokens / (ms_per_step * 1e-3), 1),
        "decode_ms": round(dec_ms, 5),
        "decode_us_per_call": round(dec_ms * 1e3, 2),
        "decode_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(dec_t, [10, 50, 90])],
        "decode_GBps": round(dec_gbs, 2),
        "pct_of_hbm_peak": round(100.0 * dec_gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": ("pa_decode_shared_prefix" if g.shared_prefix else "pa_decode") +
                      ("_fp8" if fp8 else "") +
                      (" (prefix + partition + merge kernels)" if g.shared_prefix
                       else " (partition + merge kernels)"),
            "achieved": round(dec_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(u_bytes),
        },
    }
    # the copy and scatter stages: HBM-bound bit copies, algorithmic bytes per call / mean event time
    stage_bytes = {"copy_blocks": copy_bytes(w, esize), "reshape_and_cache": scatter_bytes(w, esize)}
    if stage_us:
        out["stages"] = {}
        for name, us in stage_us.items():
            gbs = stage_bytes[name] / (us * 1e-6) / 1e9
            out["stages"][name] = {
                "us_per_call": round(us, 2), "algorithmic_bytes": int(stage_bytes[name]),
                "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if graph_ms is not None:
        out["graph"] = {
            "ms_per_step": round(graph_ms, 5),
            "value": round(step_bytes / (graph_ms * 1e-3) / 1e9, 2),
            "step_tokens_per_s": round(step_tokens / (graph_ms * 1e-3), 1),
            "decode_tokens_per_s": round(w.n_decode / (graph_ms * 1e-3), 1),
        }
    if g.shared_prefix or u_bytes != d_bytes:
        out["decode_logical_bytes"] = int(d_bytes)
        out["decode_GBps_logical"] = round(d_bytes / (dec_ms * 1e-3) / 1e9, 2)
    multi = has_prefill and g.multi_token
    if multi:
        # short chunks through pa_decode_multi: HBM-bound like a decode
        m_gbs = p_bytes / (pre_ms * 1e-3) / 1e9
        out["prefill_ms"] = round(pre_ms, 5)
        out["prefill_ms_p10_p50_p90"] = [round(float(x), 5)
                                         for x in np.percentile(pre_t, [10, 50, 90])]
        out["multi_token_rows_per_s"] = round(int(g.pre_query.shape[0]) / (ms_per_step * 1e-3), 1)
        mrec = committed_record(tag, "traffic", DECODE_SRCS)
        out["roofline_prefill"] = {
            "bound": "hbm",
            "kernel": "pa_decode_multi" + ("_fp8" if fp8 else "") + " (multi-token + merge kernels)",
            "achieved": round(m_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(m_gbs / HBM_PEAK_GBS, 4),
            "traffic": mrec.get("hbm_bytes_per_launch") if mrec and not g.n_decode else None,
            "algorithmic_bytes_per_launch": int(p_bytes), "flops_per_launch": int(p_flops)}
        if not g.n_decode:  # the multi-token kernel is the step's dominant kernel
            out["roofline"] = dict(out["roofline_prefill"])
            out["pct_of_hbm_peak"] = round(100.0 * m_gbs / HBM_PEAK_GBS, 2)
    elif has_prefill:
        out["prefill_ms"] = round(pre_ms, 5)
        out["prefill_ms_p10_p50_p90"] = [round(float(x), 5)
                                         for x in np.percentile(pre_t, [10, 50, 90])]
        out["prefill_TFLOPs"] = round(p_flops / (pre_ms * 1e-3) / 1e12, 2)
        out["prefill_mfma_frac"] = round(p_flops / (pre_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        crec = committed_record(tag, "prefill_counters", PREFILL_SRCS)
        out["roofline_prefill"] = {
            "bound": "mfma", "kernel": "pa_prefill_chunk" + ("_fp8" if fp8 else ""),
            "achieved": out["prefill_TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": out["prefill_mfma_frac"], "flops_per_launch": int(p_flops),
            # MFMA-busy share of SIMD cycles from the committed counter record of these sources
            "mfma_busy_counter": crec.get("mfma_busy_frac") if crec else None}
    if not args.no_cpu_baseline and multi and not g.n_decode:
        out["cpu_baseline"] = cpu_baseline_multi(w, args.cpu_seconds,
                                                 (args.k_scale, args.v_scale) if fp8 else None)
    elif not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds,
                                           (args.k_scale, args.v_scale) if fp8 else None)
        if has_prefill:
            out["cpu_baseline_prefill"] = cpu_baseline_prefill(
                w, args.cpu_seconds, (args.k_scale, args.v_scale) if fp8 else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
