#!/usr/bin/env python3
"""MTP round throughput on one MI355X.

Default workload (``--workload qwen35_27b_round``): the Qwen3.5-27B-shaped MTP
head (H=5120, 24/4 heads, head_dim 256, SwiGLU 17408, vocab 152064 borrowed
lm_head), bf16 weights and activations with fp32 accumulation, batch 1, draft
KV context 4096, 2 drafts per round (block_size 3), temperature 0, weights
N(0, 0.02) seeded (synthetic: no checkpoint).  One bench step is one MTP round,
the whole hot path:
  flush of the completed pairs (LAST) -> 1 chained draft step -> greedy verify of
  the 3 target rows -> draft-KV rollback (policy A) -> one host sync reading the
  accepted count, committed tokens and the KV state.
Target logits rows (N(0, 3)) and target hiddens (N(0, 1)) are synthetic inputs
drawn per round from a pool of 8 resident rounds.  Every pointer and count of a
round is device-resident, so the host enqueues round r + 1 before it waits for
round r: the round's host synchronisation overlaps the next round's GPU work.
--graph replays each round from a HIP graph instead.

Other workloads (one JSON line each, same keys):
  tiny_round            the tiny fp32 head (H 256), prefix 128, 2 drafts, 64 rounds
  flush256_prefix8192   the 256-pair flush (tiny head in bf16) after an 8192-slot
                        prefix, ALL mode, the KV rolled back after each flush
  flush256_qwen35_27b   the same flush at the 27B shape after 4096 slots (the
                        pages' 2.5 MiB flush cap; MFMA GEMM roofline)
  verify_sampled        sampled verification: N=4, V=152064, T 0.7, penalty 1.1
                        over a 64-token ring, top-k 40 (--top-k; 0 = the whole
                        vocabulary), top-p 0.9, min-p 0.05
  depth_ctx32768        rounds of the tiny bf16 head over a 32768-slot prefix at
                        depth --depth (1..8), lm_head bf16 or int8-g128 (--lm),
                        planted acceptance p_i = 0.8 * 0.85^i, policy A or B,
                        --sessions independent sessions rotated (cold KV)
  launch_floor          back-to-back launches of the one-workgroup KV rollback:
                        the GPU time of one dependent launch (eager and graph)
  batch_qwen35_27b      --batch (default 4) independent sessions of the 27B-shaped
                        head, 4096-slot prefixes, 2 drafts, greedy, in batched calls
                        (each weight streamed once for every session's rows)

Each line carries ``roofline`` for the workload's dominant kernel (algorithmic
bytes or flops per launch / its average duration from HIP events recorded
around each launch inside the timed region) and ``cpu_baseline`` (the fp64 numpy
oracle timed on a bounded sample of the same workload on the host).
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MTP draft tokens/sec + verify rounds/sec at batch 1 (GB/s vs HBM peak)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
VALU_FP32_PEAK_TFLOPS = 157.3
POOL = 8
TIME_EVERY = 8     # rounds between the ones whose dominant kernel carries timing events


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes and flops
# ---------------------------------------------------------------------------
def _bytes_of(dtype):
    return {"bf16": 2, "f32": 4, "i8g128": 1}[dtype]


def step_bytes(shape, ctx_len, with_logits=False):
    """Algorithmic HBM bytes of one draft-head step at KV length ctx_len (the new
    slot included): every weight once, one embedding row, the KV read and the new
    K/V row written, the hidden in/out, plus logits if they are written."""
    H, D, hkv, V = shape.hidden, shape.head_dim, shape.n_kv_heads, shape.vocab
    wb, kvb, ab = _bytes_of(shape.weight_dtype), _bytes_of(shape.kv_dtype), _bytes_of(shape.act_dtype)
    head = shape.head_param_count() * wb
    lm = V * H * _bytes_of(shape.lm_head_dtype)
    if shape.lm_head_dtype == "i8g128":
        lm += V * (H // 128) * 2
    kv = 2 * hkv * D * kvb * ctx_len
    return head + lm + H * wb + kv + 2 * H * ab + (V * 4 if with_logits else 0)


def unembed_bytes(shape):
    """Algorithmic bytes of one unembedding launch: the lm_head (plus its scales),
    the fp32 input vector, the final-norm weight (logits are not written in the
    timed rounds)."""
    H, V = shape.hidden, shape.vocab
    extra = V * (H // 128) * 2 if shape.lm_head_dtype == "i8g128" else 0
    return V * H * _bytes_of(shape.lm_head_dtype) + extra + H * 4 + H * _bytes_of(shape.weight_dtype)


def attention_bytes(shape, keys, rows=1):
    """Algorithmic bytes of one attention launch: the K and V of ``keys`` slots
    (read once per kv head), the fp32 roped q read and the fp32 o written per row."""
    kvb = _bytes_of(shape.kv_dtype)
    return 2 * shape.n_kv_heads * shape.head_dim * kvb * keys + rows * 2 * shape.n_q_heads * shape.head_dim * 4


def flush_attention_flops(shape, prefix, n):
    """Causal attention flops of an n-row flush after `prefix` slots: row j
    attends over prefix + j + 1 keys, 4 D flops per key per query head (q.k and
    p.v)."""
    keys = n * (prefix + 1) + n * (n - 1) // 2
    return 4 * shape.head_dim * shape.n_q_heads * keys


def flush_projection_flops(shape, n, rows_out):
    """Projection flops of a flush: fc and q/k/v for every row; o, gate/up, down
    for the rows whose output is requested; the unembedding of the last row."""
    H, D, I = shape.hidden, shape.head_dim, shape.intermediate
    qkv = (shape.n_q_heads + 2 * shape.n_kv_heads) * D * H
    per_out = shape.n_q_heads * D * H + 3 * H * I
    return 2 * (n * (2 * H * H + qkv) + rows_out * per_out + shape.vocab * H)


# ---------------------------------------------------------------------------
# measured HBM traffic (rocprofv3 PMC summaries committed under profiles/)
# ---------------------------------------------------------------------------
def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mtp_draft_head_step_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# the sources of the unembedding GEMV launch (kernel template, its bf16
# single-row instantiation, the dispatch, shared headers)
UNEMBED_SOURCES = ("gemv_impl.h", "gemv_bf16_1.hip", "gemv.hip", "common.h", "kernels.h")


def gemv_source_digest():
    return source_digest(UNEMBED_SOURCES)


def measured_traffic(name, files):
    """HBM bytes per launch from a committed PMC summary profiles/<name>.json, or
    None if there is none or the kernel's sources changed since it was taken."""
    p = os.path.join(ROOT, "profiles", name + ".json")
    try:
        with open(p) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("source_digest", d.get("gemv_source_digest")) != source_digest(files):
        return None
    return d.get("bytes_per_launch")


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def single_thread_blas():
    """Context limiting BLAS to one thread (the small oracle products)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except Exception:
        return contextlib.nullcontext()


def timed_sample(unit_fn, seconds, max_units):
    """Run oracle units until `seconds` of CPU time have passed (at least one,
    at most max_units); returns (units, elapsed seconds)."""
    t = time.perf_counter()
    n = 0
    while n < max_units:
        unit_fn(n)
        n += 1
        if time.perf_counter() - t >= seconds:
            break
    return n, time.perf_counter() - t


def host_info():
    """The host the oracle baseline runs on: CPU model, logical CPUs, 1-minute load."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpus": os.cpu_count(), "load_1m": round(os.getloadavg()[0], 2)}


def with_host(cpu):
    """A cpu_baseline entry with the host's CPU model and load added."""
    if cpu is not None:
        h = host_info()
        cpu.update({"cpu_model": h["cpu_model"], "host_cpus": h["cpus"], "load_1m": h["load_1m"]})
    return cpu


def spread(values, digits=3):
    """Median of repeated measurements with their min and max (the pages' method:
    each arm run several times, median reported with its range)."""
    import statistics
    return {"median": round(statistics.median(values), digits), "min": round(min(values), digits),
            "max": round(max(values), digits), "n": len(values)}


def roofline(bound, achieved, peak, unit, traffic, **extra):
    if achieved is None:
        return None
    d = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    d.update(extra)
    return d


def base_line(args, value, unit, ms_step, dtype, data, config):
    return {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": data, "config": config}


def calibrate_copy(args):
    """Three 1 GiB device-to-device copies: a plain copy kernel of known size,
    for scaling HBM traffic counters."""
    if not args.calibrate_copy:
        return
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# the round's results on the host
# ---------------------------------------------------------------------------
class HostRows:
    """`rows` x `cols` int32 rows in host-coherent pinned memory, each written
    by a round's final verify kernel (system-scope stores, no copy launch), with
    one completion event per row.  Those stores reach host memory uncached, so
    the events are created without the system-scope fence (an event with it
    writes back and invalidates the GPU's L2 between every two rounds).  The
    HIP calls go to the runtime libmtp is bound to (symbol lookup through its
    handle)."""
    COHERENT = 0x40000000                                           # hipHostMallocCoherent
    EV_FLAGS = 0x2 | 0x20000000                                     # DisableTiming | DisableSystemFence

    def __init__(self, rows, cols):
        import ctypes as C
        from mtp_draft_head_step_amd import abi
        import numpy as np
        self.C, hip = C, C.CDLL(abi.LIB_PATH)
        vp = C.c_void_p
        hip.hipHostMalloc.argtypes = [C.POINTER(vp), C.c_size_t, C.c_uint]
        hip.hipHostFree.argtypes = [vp]
        hip.hipEventCreateWithFlags.argtypes = [C.POINTER(vp), C.c_uint]
        hip.hipEventRecord.argtypes = [vp, vp]
        hip.hipEventSynchronize.argtypes = [vp]
        hip.hipEventDestroy.argtypes = [vp]
        self.hip, self.rows, self.cols = hip, rows, cols
        self.ptr = vp()
        self._ok(hip.hipHostMalloc(C.byref(self.ptr), rows * cols * 4, self.COHERENT), "hipHostMalloc")
        self.view = np.ctypeslib.as_array((C.c_int32 * (rows * cols)).from_address(self.ptr.value)).reshape(rows, cols)
        self.view[:] = 0
        self.ev = []
        for _ in range(rows):
            e = vp()
            self._ok(hip.hipEventCreateWithFlags(C.byref(e), self.EV_FLAGS), "hipEventCreateWithFlags")
            self.ev.append(e)

    @staticmethod
    def _ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def addr(self, i):
        """Host address of row i: the report row the round's final verify
        kernel writes (spec_verify_rollback)."""
        return self.ptr.value + i * self.cols * 4

    def record(self, i, stream):
        self._ok(self.hip.hipEventRecord(self.ev[i], stream.cuda_stream), "hipEventRecord")

    def wait(self, i):
        self._ok(self.hip.hipEventSynchronize(self.ev[i]), "hipEventSynchronize")
        return self.view[i]

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []
        if self.ptr.value:
            self.hip.hipHostFree(self.ptr)
            self.ptr = self.C.c_void_p()
            self.view = None


# ---------------------------------------------------------------------------
# greedy rounds (the 27B-shaped head; the tiny fp32 head)
# ---------------------------------------------------------------------------
def run_greedy_rounds(args, shape, wl, ctx, N, workload, data, use_graphs=False):
    import numpy as np
    import torch

    from mtp_draft_head_step_amd import abi
    from mtp_draft_head_step_amd import inputs as I

    V, H = shape.vocab, shape.hidden
    t0 = time.time()
    storage = I.head_weights(shape, wl)
    log(f"weights generated in {time.time() - t0:.1f}s")
    head = abi.Head(shape, storage)
    cap = ctx + 1 + (args.warmup + 2 * args.repeats * args.steps + POOL + 4) * (N + 1) + 64
    kp, vp = I.prefix_kv(shape, wl, ctx, cap)
    # one device buffer {KV state words | k, k+1, committed tokens}: the round's
    # results reach the host in one copy
    iost = torch.zeros(4 + 2 + N + 1, dtype=torch.int32, device="cuda")
    kv = abi.DraftKV(shape, cap, kp, vp, ctx, state=iost[0:4])
    pool_logits = np.stack([I.logits_rows(wl, 5, r, N + 1, V, 3.0)[0] for r in range(POOL)])
    pool_hid = np.stack([I.target_hiddens(shape, wl, r, N + 1) for r in range(POOL)])
    first_tok = I.tokens_uniform(wl, 0, N + 1, V)
    first_hid = I.target_hiddens(shape, wl, 1000, N + 1)
    ring0, ring_st0 = I.history_ring(wl, None, 64, V)
    act = torch.bfloat16 if shape.act_dtype == I.BF16 else torch.float32
    t_logits = abi.to_device(pool_logits)
    t_hid = abi.to_device(pool_hid)
    ring = abi.to_device(ring0)
    ring_st = abi.to_device(ring_st0)
    io = iost[4:]                                                      # {k, k+1, tokens...}
    d_buf = torch.zeros(N, dtype=torch.int32, device="cuda")
    g_buf = torch.zeros((N, H), dtype=act, device="cuda")
    ws = abi.Workspace(abi.mtp_workspace_bytes(head.cfg, N + 1, cap))
    vws = abi.Workspace(abi.spec_verify_workspace_bytes(N, V))
    sp = abi.sampling(window=64)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"inputs resident ({(time.time() - t0):.1f}s); capacity {cap}")

    # Pending pairs live in fixed places so every round has the same pointers:
    # tokens = io[2:] (written by the previous verify), count = io[1], hiddens =
    # the previous round's target hiddens.  Round 0 starts from one pending pair.
    io[1] = 1
    io[2:] = abi.to_device(first_tok)
    t_hid[POOL - 1].copy_(abi.to_device(first_hid))
    host = HostRows(POOL, iost.numel())
    totals = {"committed": 0, "accepted": 0, "rounds": 0}
    last = {}

    def enqueue_round(r, st):
        prev = (r - 1) % POOL
        # flush of the pending pairs + N - 1 chained steps, one call
        abi.mtp_draft_chain(head, kv, io[2:], t_hid[prev], N + 1, io[1:2], N, d_buf, g_buf, None, ws, st)
        # verify, the rollback to the round base (policy A) and the round's
        # results for the host (KV state words, k, k+1, tokens) in one call
        abi.spec_verify_rollback(sp, N, V, t_logits[r % POOL], None, d_buf, ring, ring_st, None, io[2:], io[0:2],
                                 vws, kv, abi.TO_ROUND_BASE, False, host.addr(r % POOL), st)

    def consume(r):
        row = host.view[r % POOL]
        if int(row[3]) != 0:
            raise RuntimeError(f"device error word {int(row[3])} in round {r}")
        # each round flushes the previous round's committed pairs and rolls back
        # to that base: a stale row would break this chain
        if last and int(row[0]) != last["len"] + last["committed"]:
            raise RuntimeError(f"round {r}: KV length {int(row[0])}, expected {last['len'] + last['committed']}")
        last.update(len=int(row[0]), committed=int(row[5]))
        totals["committed"] += int(row[5])
        totals["accepted"] += int(row[4])
        totals["rounds"] += 1

    for r in range(args.warmup):                       # eager rounds
        enqueue_round(r, stream)
        stream.synchronize()
        consume(r)
    log(f"warmup {args.warmup} rounds done")

    def repeat(graphs, first):
        """One timed repeat of args.steps rounds starting at round `first`;
        returns its elapsed seconds."""
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        prev = None
        for r in range(first, first + args.steps):
            if graphs is not None:
                graphs[r % POOL].replay()
            else:
                if r % TIME_EVERY == 0 or r == first:
                    abi.mtp_timing_pause(False)
                enqueue_round(r, stream)
                abi.mtp_timing_pause(True)
            host.record(r % POOL, stream)
            if prev is not None:                          # the one host sync per round,
                host.wait(prev % POOL)                    # overlapped with the next round
                consume(prev)
            prev = r
        host.wait(prev % POOL)
        consume(prev)
        torch.cuda.synchronize()
        return time.perf_counter() - t_start

    host0 = host_info()
    eager_el, graph_el = [], []
    r0 = args.warmup
    if not args.graph:
        abi.mtp_timing_begin(abi.TIME_UNEMBED, args.repeats * args.steps * N + 4)
        for _ in range(args.repeats):
            eager_el.append(repeat(None, r0))
            r0 += args.steps
        lm_ms, lm_n = abi.mtp_timing_end()
    else:
        lm_ms, lm_n = 0.0, 0
    if args.graph or use_graphs:
        # one graph per pool slot, replayed round by round (every pointer of a
        # round is fixed; the counts and tokens are device-resident)
        cap_stream = torch.cuda.Stream()
        graphs = {}
        for p_ in range(POOL):
            r = r0 + p_
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap_stream):
                enqueue_round(r, torch.cuda.current_stream())
            graphs[r % POOL] = g
        torch.cuda.synchronize()
        log("captured %d round graphs" % POOL)
        for _ in range(args.repeats):
            graph_el.append(repeat(graphs, r0))
            r0 += args.steps
    host1 = host_info()
    host.close()
    els = graph_el if graph_el else eager_el
    elapsed = sorted(els)[len(els) // 2]                 # the median repeat
    log(f"timed {args.repeats} x {args.steps} rounds; median {elapsed * 1e3:.1f} ms; unembedding {lm_n} launches")
    calibrate_copy(args)

    rounds_s = args.steps / elapsed
    lm_avg_s = lm_ms / lm_n / 1e3 if lm_n else None
    ub = unembed_bytes(shape)
    round_bytes = N * step_bytes(shape, ctx + 2) + (N + 1) * V * 4
    traffic = measured_traffic("unembed_qwen35_27b_traffic", UNEMBED_SOURCES) \
        if workload == "qwen35_27b_mtp_head_round" else None

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_rounds(shape, storage, kp, vp, cap, ctx, N, pool_logits, pool_hid, first_tok, first_hid,
                         ring0, ring_st0, args.cpu_seconds, args.steps + args.warmup, single=shape.hidden < 1024)

    dtype = "bf16" if shape.weight_dtype == I.BF16 else "f32"
    out = base_line(args, round(N * rounds_s, 2), "draft tokens/s", elapsed / args.steps * 1e3, dtype, data,
                    {"workload": workload, "hidden": H, "heads": f"{shape.n_q_heads}q/{shape.n_kv_heads}kv",
                     "head_dim": shape.head_dim, "intermediate": shape.intermediate, "vocab": V,
                     "draft_kv_context": ctx, "drafts_per_round": N, "block_size": N + 1,
                     "temperature": 0.0, "batch": 1, "policy": "A", "lm_head": shape.lm_head_dtype})
    out.update({
        "rounds_per_s": round(rounds_s, 2),
        "round_gbs": round(round_bytes / (elapsed / args.steps) / 1e9, 1),
        "round_hbm_frac": round(round_bytes / (elapsed / args.steps) / 1e9 / HBM_PEAK_GBS, 4),
        "repeats": {"draft_tokens_per_s": spread([N * args.steps / e for e in els], 2),
                    "ms_per_round": spread([e / args.steps * 1e3 for e in els], 4)},
        "eager_draft_tokens_per_s": spread([N * args.steps / e for e in eager_el], 2) if eager_el else None,
        "committed_per_round": round(totals["committed"] / max(1, totals["rounds"]), 4),
        "launch": ("hip graph per round" if graph_el else "eager") +
                  ", host sync per round overlapped with the next round",
        "host": {"before": host0, "after": host1},
        "roofline": roofline("hbm", ub / lm_avg_s / 1e9 if lm_avg_s else None, HBM_PEAK_GBS, "GB/s", traffic,
                             kernel=f"unembedding GEMV (lm_head {V}x{H} {shape.lm_head_dtype})",
                             bytes_per_launch=ub, avg_us=round(lm_avg_s * 1e6, 2) if lm_avg_s else None,
                             launches=lm_n),
        "cpu_baseline": with_host(cpu),
    })
    return out


def run_launch_floor(args):
    """Back-to-back launches of the library's smallest kernel (the one-workgroup
    KV rollback, which loads the state words and stores the length): the GPU
    time one dependent launch costs on its stream, eagerly and replayed from a
    HIP graph.  Every small kernel of a round pays about this much."""
    import torch

    from mtp_draft_head_step_amd import abi
    from mtp_draft_head_step_amd import inputs as I

    shape = I.TINY_BF16
    kp, vp = I.prefix_kv(shape, I.WL_TINY, 16, 64)
    kv = abi.DraftKV(shape, 64, kp, vp, 16)
    stream = torch.cuda.current_stream()
    per = 256                                          # launches per timed batch

    def batch():
        st = torch.cuda.current_stream()            # the capture stream inside the graph block
        for _ in range(per):
            abi.kv_rollback(kv, 16, None, 0, st)      # to the current length: a no-op

    for _ in range(args.warmup):
        batch()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap_stream):
        batch()
    torch.cuda.synchronize()
    eager, graph = [], []
    for _ in range(args.repeats):
        for mode, out in (("eager", eager), ("graph", graph)):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            ev[0].record(stream)
            for _ in range(args.steps):
                if mode == "eager":
                    batch()
                else:
                    g.replay()
            ev[1].record(stream)
            torch.cuda.synchronize()
            out.append(ev[0].elapsed_time(ev[1]) * 1e3 / (args.steps * per))
    if int(kv.state[3].item()) != 0 or int(kv.state[0].item()) != 16:
        raise RuntimeError("device error word set by the launch-floor kernels")
    e_med = sorted(eager)[len(eager) // 2]
    g_med = sorted(graph)[len(graph) // 2]
    line = base_line(args, round(1e6 / g_med, 1), "launches/s", round(g_med * 1e-3, 6), "int32",
                     "synthetic (a 64-slot tiny-head draft KV; the launches change nothing)",
                     {"workload": "launch_floor_one_workgroup", "kernel": "KV rollback to the current length",
                      "launches_per_batch": per})
    line["us_per_launch"] = {"graph": spread(graph), "eager": spread(eager)}
    line["higher_is_better"] = True
    line["roofline"] = None
    line["cpu_baseline"] = None
    return line


# ---------------------------------------------------------------------------
# B sessions per round (the 27B-shaped head): one weight pass for every session
# ---------------------------------------------------------------------------
def run_batch_rounds(args):
    """Greedy rounds of --batch independent sessions of the 27B-shaped head,
    each at a 4096-slot prefix, launched as batched calls: mtp_draft_chain_batch
    (the pending pairs of every session flushed, then the chained step, each
    weight streamed once for all sessions' rows), spec_verify_batch,
    kv_rollback_batch (policy A); one host sync per round (the sessions' state
    words and counts), overlapped with the next round."""
    import numpy as np
    import torch

    from mtp_draft_head_step_amd import abi
    from mtp_draft_head_step_amd import inputs as I

    B, N, ctx = int(args.batch), 2, 4096
    if not 1 <= B <= 16:
        raise SystemExit("--batch takes 1..16 sessions")
    shape, wl = I.QWEN35_27B, I.WL_QWEN
    V, H = shape.vocab, shape.hidden
    t0 = time.time()
    storage = I.head_weights(shape, wl)
    head = abi.Head(shape, storage)
    cap = ctx + 1 + (args.warmup + args.repeats * args.steps + POOL + 4) * (N + 1) + 64
    kps, vps = zip(*[I.prefix_kv(shape, wl + 100 * b, ctx, cap) for b in range(B)])
    kv = abi.BatchKV(shape, B, cap, np.stack(kps), np.stack(vps), [ctx] * B)
    del kps, vps
    pool_logits = np.stack([np.stack([I.logits_rows(wl, 5, (r, b), N + 1, V, 3.0)[0] for b in range(B)])
                            for r in range(POOL)])
    pool_hid = np.stack([np.stack([I.target_hiddens(shape, wl, (r, b), N + 1) for b in range(B)])
                         for r in range(POOL)])
    t_logits, t_hid = abi.to_device(pool_logits), abi.to_device(pool_hid)
    i32 = dict(dtype=torch.int32, device="cuda")
    rings = [I.history_ring(wl, b, 64, V) for b in range(B)]
    ring = abi.to_device(np.stack([r for r, _ in rings]))
    ring_st = abi.to_device(np.stack([st for _, st in rings]))
    # pending pairs live in fixed places: tokens = out_t (the previous verify's
    # committed tokens), count = out_c[:, 1], hiddens = the previous round's
    # target hiddens; round 0 starts from one pending pair per session
    out_t = abi.to_device(np.stack([I.tokens_uniform(wl, (0, b), N + 1, V) for b in range(B)]).astype(np.int32))
    out_c = torch.zeros((B, 2), **i32)
    out_c[:, 1] = 1
    t_hid[POOL - 1].copy_(abi.to_device(np.stack([I.target_hiddens(shape, wl, (1000, b), N + 1)
                                                  for b in range(B)])))
    d_buf = torch.zeros((B, N), **i32)
    g_buf = torch.zeros((B, N, H), dtype=torch.bfloat16, device="cuda")
    ws = abi.Workspace(abi.mtp_batch_workspace_bytes(head.cfg, B, N + 1, cap))
    vws = abi.Workspace(B * abi.spec_verify_workspace_bytes(N, V))
    sp = abi.sampling(window=64)
    host_st = torch.zeros((POOL, B, 4), dtype=torch.int32).pin_memory()
    host_c = torch.zeros((POOL, B, 2), dtype=torch.int32).pin_memory()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"{B} sessions resident ({time.time() - t0:.1f}s); capacity {cap}")
    totals = {"committed": 0, "rounds": 0}
    last = {}

    def enqueue_round(r, st):
        prev = (r - 1) % POOL
        abi.mtp_draft_chain_batch(head, kv, B, out_t, t_hid[prev], N + 1, out_c[:, 1:], 2, N, d_buf, g_buf, None,
                                  ws, st)
        abi.spec_verify_batch(sp, B, N, V, t_logits[r % POOL], None, d_buf, ring, ring_st, None, out_t, out_c,
                              vws, st)
        abi.kv_rollback_batch(kv, B, abi.TO_ROUND_BASE, None, N, st)
        host_st[r % POOL].copy_(kv.state, non_blocking=True)
        host_c[r % POOL].copy_(out_c, non_blocking=True)

    def consume(r):
        sw, cw = host_st[r % POOL], host_c[r % POOL]
        if int(sw[:, 3].abs().sum()) != 0:
            raise RuntimeError(f"device error words {sw[:, 3].tolist()} in round {r}")
        lens, comm = sw[:, 0].tolist(), cw[:, 1].tolist()
        if last and [a + c for a, c in zip(last["len"], last["comm"])] != lens:
            raise RuntimeError(f"round {r}: KV lengths {lens} do not follow the previous round")
        last.update(len=lens, comm=comm)
        totals["committed"] += sum(comm)
        totals["rounds"] += 1

    for r in range(args.warmup):
        enqueue_round(r, stream)
        stream.synchronize()
        consume(r)
    els = []
    r0 = args.warmup
    abi.mtp_timing_begin(abi.TIME_UNEMBED, args.repeats * args.steps * N + 4)
    for _ in range(args.repeats):
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        done = [torch.cuda.Event(), torch.cuda.Event()]
        prev = None
        for r in range(r0, r0 + args.steps):
            abi.mtp_timing_pause(not (r % TIME_EVERY == 0 or r == r0))
            enqueue_round(r, stream)
            abi.mtp_timing_pause(True)
            done[r % 2].record(stream)
            if prev is not None:
                done[prev % 2].synchronize()
                consume(prev)
            prev = r
        done[prev % 2].synchronize()
        consume(prev)
        torch.cuda.synchronize()
        els.append(time.perf_counter() - t_start)
        r0 += args.steps
    lm_ms, lm_n = abi.mtp_timing_end()
    elapsed = sorted(els)[len(els) // 2]
    rounds_s = args.steps / elapsed
    # three sessions and more with a bf16 lm_head: one matrix-core product over
    # the sessions' last rows (the lm_head read once); else GEMV launches of four
    product = B >= 3 and shape.lm_head_dtype == I.BF16
    groups = 1 if product else (B + 3) // 4
    ub = unembed_bytes(shape) * groups
    ukind = (f"unembedding product over the {B} sessions' last rows (one matrix-core launch, lm_head {V}x{H} "
             f"bf16)" if product else
             f"unembedding GEMV ({B} rows in {groups} launch(es) of up to four, lm_head {V}x{H} bf16)")
    lm_avg_s = lm_ms / lm_n / 1e3 if lm_n else None
    cpu = None
    if args.cpu_seconds > 0:
        # the oracle runs sessions one after another: session 0's rounds give its rate
        kp0, vp0 = I.prefix_kv(shape, wl, ctx, cap)
        cpu = cpu_rounds(shape, storage, kp0, vp0, cap, ctx, N, pool_logits[:, 0], pool_hid[:, 0],
                         I.tokens_uniform(wl, (0, 0), N + 1, V), I.target_hiddens(shape, wl, (1000, 0), N + 1),
                         rings[0][0], rings[0][1], args.cpu_seconds, args.steps + args.warmup, single=False)
        cpu["sample"] = ("session 0 of the batch: " + cpu["sample"] +
                         "; the oracle runs the sessions one after another, so its rate does not depend on B")
    out = base_line(args, round(B * N * rounds_s, 2), "draft tokens/s", elapsed / args.steps * 1e3, "bf16",
                    "synthetic (seeded N(0,0.02) weights of the Qwen3.5-27B MTP head shape; per session a "
                    "4096-slot N(0,1) prefix, N(0,3) target logits, N(0,1) target hiddens)",
                    {"workload": "qwen35_27b_mtp_head_round_batch", "sessions": B, "hidden": H,
                     "heads": f"{shape.n_q_heads}q/{shape.n_kv_heads}kv", "head_dim": shape.head_dim,
                     "intermediate": shape.intermediate, "vocab": V, "draft_kv_context": ctx,
                     "drafts_per_round": N, "temperature": 0.0, "policy": "A", "lm_head": shape.lm_head_dtype})
    out.update({
        "rounds_per_s": round(rounds_s, 2),
        "draft_tokens_per_s_per_session": round(N * rounds_s, 2),
        "repeats": {"draft_tokens_per_s": spread([B * N * args.steps / e for e in els], 2),
                    "ms_per_round": spread([e / args.steps * 1e3 for e in els], 4)},
        "committed_per_round": round(totals["committed"] / max(1, totals["rounds"]), 4),
        "launch": "eager, batched calls, host sync per round overlapped with the next round",
        "roofline": roofline("hbm", ub / lm_avg_s / 1e9 if lm_avg_s else None, HBM_PEAK_GBS, "GB/s", None,
                             kernel=ukind, bytes_per_launch=ub,
                             avg_us=round(lm_avg_s * 1e6, 2) if lm_avg_s else None, launches=lm_n),
        "cpu_baseline": with_host(cpu),
    })
    return out


def cpu_rounds(shape, storage, kp, vp, cap, ctx, N, pool_logits, pool_hid, first_tok, first_hid, ring0,
               ring_st0, seconds, max_rounds, single):
    """The oracle as it stands, on the host: `rounds` rounds of the same workload."""
    from mtp_draft_head_step_amd import inputs as I
    from oracle import head as OH
    from oracle import rounds as OR
    from oracle.kvcache import DraftKV
    t0 = time.time()
    oh = OH.Head(shape, I.weight_values(shape, storage))
    okv = DraftKV(shape.n_kv_heads, cap, shape.head_dim, I.decode(kp, shape.kv_dtype),
                  I.decode(vp, shape.kv_dtype), ctx)
    pending = [(int(first_tok[0]), I.decode(first_hid[0], shape.act_dtype))]
    st = OR.RoundState(oh, okv, pending, [0] * (ctx + 2), ring0, ring_st0, window=64)
    log(f"oracle inputs decoded in {time.time() - t0:.1f}s")

    def target_fn(toks, start):
        r = target_fn.r
        return pool_logits[r % POOL], I.decode(pool_hid[r % POOL], shape.act_dtype)

    def unit(r):
        target_fn.r = r
        OR.run_round(st, N, target_fn, policy="A")
    with (single_thread_blas() if single else contextlib.nullcontext()):
        cores = 1 if single else cpu_threads()
        rounds, el = timed_sample(unit, seconds, max_rounds)
    log(f"oracle {rounds} round(s) in {el:.1f}s")
    return {"value": round(N * rounds / el, 4), "unit": "draft tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{rounds} round(s) of the same workload (flush + {N - 1} chained step(s) + greedy verify "
                      f"+ rollback at draft KV context {ctx}), numpy fp64"}


# ---------------------------------------------------------------------------
# the 256-pair flush
# ---------------------------------------------------------------------------
def run_flush(args, big=False):
    """The 256-pair flush in ALL mode: the tiny head in bf16 after 8192 slots, or
    (big) the 27B-shaped head after 4096 slots (256 x 5120 bf16 pending hiddens,
    the pages' 2.5 MiB flush cap).  Timed with a rollback to the prefix after
    each flush."""
    import torch

    from mtp_draft_head_step_amd import abi
    from mtp_draft_head_step_amd import inputs as I

    if big:
        shape, wl, prefix = I.QWEN35_27B, I.WL_QWEN, 4096
    else:
        shape, wl, prefix = I.TINY_BF16, I.WL_FLUSH, 8192
    n = 256
    cap = prefix + n
    storage = I.head_weights(shape, wl)
    head = abi.Head(shape, storage)
    kp, vp = I.prefix_kv(shape, wl, prefix, cap)
    kv = abi.DraftKV(shape, cap, kp, vp, prefix)
    toks_np = I.tokens_uniform(wl, 0, n, shape.vocab)
    hids_np = I.target_hiddens(shape, wl, 0, n)
    toks, hids = abi.to_device(toks_np), abi.to_device(hids_np)
    ws = abi.Workspace(abi.mtp_workspace_bytes(head.cfg, n, cap))
    hout = torch.zeros((n, shape.hidden), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    amax = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def flush(mode, st=None):
        st = stream if st is None else st
        abi.mtp_flush_pairs(head, kv, toks, hids, n, None, mode, 1, hout if mode == abi.ALL else hout[:1],
                            logits, amax, ws, st)
        abi.kv_rollback(kv, prefix, None, 0, st)

    def timed(mode, steps, kind=None):
        for _ in range(args.warmup):
            flush(mode)
        torch.cuda.synchronize()
        if kind is not None:
            abi.mtp_timing_begin(kind, 64 * steps + 4)
        t = time.perf_counter()
        for i in range(steps):
            if kind is not None:
                abi.mtp_timing_pause(i % TIME_EVERY != 0)
            flush(mode)
        torch.cuda.synchronize()
        el = time.perf_counter() - t
        k = abi.mtp_timing_end() if kind is not None else None
        if int(kv.state[3].item()) != 0:
            raise RuntimeError("device error word set")
        return el / steps, k

    side = max(args.steps // 4, 5)
    timed_side = (side + TIME_EVERY - 1) // TIME_EVERY      # flushes carrying timing events
    t_all, (att_ms, att_n) = timed(abi.ALL, args.steps, abi.TIME_ATTENTION)
    _, (proj_ms, proj_n) = timed(abi.ALL, side, abi.TIME_PROJECTION)
    t_last, _ = timed(abi.LAST, side)
    t_kv, _ = timed(abi.KV_ONLY, side)
    # the same ALL-mode flush (and its rollback) replayed from one HIP graph:
    # no host launch gaps between its kernels
    graph = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap_stream):
        flush(abi.ALL, torch.cuda.current_stream())
    torch.cuda.synchronize()
    g_els = []
    for _ in range(args.repeats):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        g_els.append((time.perf_counter() - t) / args.steps)
    if int(kv.state[3].item()) != 0:
        raise RuntimeError("device error word set")
    t_graph = sorted(g_els)[len(g_els) // 2]
    calibrate_copy(args)
    att_flops = flush_attention_flops(shape, prefix, n)
    proj_flops = flush_projection_flops(shape, n, n)
    gemm_flops = proj_flops - 2 * shape.vocab * shape.hidden      # the last row's unembedding is a GEMV
    total_flops = att_flops + proj_flops
    att_avg = att_ms / att_n / 1e3
    proj_s = proj_ms / timed_side / 1e3                             # the GEMMs of one flush
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_flush(shape, storage, kp, vp, cap, prefix, toks_np, hids_np, args.cpu_seconds, args.steps,
                        cache_fp64=big)
    heads = f"{shape.n_q_heads}q/{shape.n_kv_heads}kv"
    name = "flush256_qwen35_27b_prefix4096" if big else "flush256_prefix8192"
    out = base_line(args, round(n / t_graph, 1), "flushed pairs/s", t_graph * 1e3, "bf16",
                    f"synthetic (seeded N(0,0.02) weights of the {'Qwen3.5-27B-shaped' if big else 'tiny'} head "
                    "in bf16; 256 uniform tokens, N(0,1) bf16 hiddens; N(0,1) bf16 prefix K/V)",
                    {"workload": name, "hidden": shape.hidden, "heads": heads, "head_dim": shape.head_dim,
                     "intermediate": shape.intermediate, "vocab": shape.vocab, "pairs": n,
                     "prefix": prefix, "mode": "ALL (every row's g; last row's logits and argmax)"})
    if big:   # the projections dominate: the roofline is the MFMA GEMMs of one flush
        line = roofline("mfma", gemm_flops / proj_s / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", None,
                        kernel="the flush's five MFMA products (fc, qkv, o, gate/up, down; all 256 rows per workgroup, weights streamed once; split-K reduce included)",
                        flops_per_launch=round(gemm_flops / max(1, proj_n // timed_side)),
                        avg_us=round(proj_s * 1e6 / max(1, proj_n // timed_side), 2), launches=proj_n)
    else:     # the attention dominates
        line = roofline("mfma", att_flops / att_avg / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", None,
                        kernel="causal flush attention on bf16 MFMA (256 rows x 4 q heads over "
                               "8193..8448 keys; split-K partials)",
                        flops_per_launch=att_flops, avg_us=round(att_avg * 1e6, 2), launches=att_n)
    out.update({
        "launch": "one HIP graph per flush (with its rollback to the prefix), replayed",
        "repeats": {"flush_us": spread([t * 1e6 for t in g_els], 2)},
        "flush_us": {"all_graph": round(t_graph * 1e6, 2), "all_eager": round(t_all * 1e6, 2),
                     "last_eager": round(t_last * 1e6, 2), "kv_only_eager": round(t_kv * 1e6, 2)},
        "flush_tflops": round(total_flops / t_graph / 1e12, 3),
        "flush_mfma_frac": round(total_flops / t_graph / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
        "algorithmic_gflop": {"attention": round(att_flops / 1e9, 4), "projections": round(proj_flops / 1e9, 4)},
        "attention_us": round(att_avg * 1e6, 2),
        "attention_tflops": round(att_flops / att_avg / 1e12, 2),
        "projection_us_per_flush": round(proj_s * 1e6, 2),
        "projection_tflops": round(gemm_flops / proj_s / 1e12, 2),
        "projection_launches_per_flush": proj_n // timed_side,
        "roofline": line,
        "cpu_baseline": with_host(cpu),
    })
    return out


def run_flush_scaling(args):
    """Flush cost against its size at the 27B shape: n = 1..256 pending pairs
    after 4096 slots, in LAST mode (the in-round use: every row's K/V, the last
    row's g, logits and argmax) and in KV_ONLY mode.  A flush of one pair is one
    draft step; the curve says how much less than n steps' price n positions
    cost.  The line's value and roofline are the 256-pair LAST flush's."""
    import torch

    from mtp_draft_head_step_amd import abi
    from mtp_draft_head_step_amd import inputs as I

    shape, wl, prefix = I.QWEN35_27B, I.WL_QWEN, 4096
    sizes = sorted({int(x) for x in str(args.rows).split(",")})
    if not sizes or sizes[0] < 1 or sizes[-1] > 256:
        raise SystemExit("--rows: pair counts in 1..256")
    nmax = sizes[-1]
    cap = prefix + nmax
    storage = I.head_weights(shape, wl)
    head = abi.Head(shape, storage)
    del storage
    kp, vp = I.prefix_kv(shape, wl, prefix, cap)
    kv = abi.DraftKV(shape, cap, kp, vp, prefix)
    toks = abi.to_device(I.tokens_uniform(wl, 0, nmax, shape.vocab))
    hids = abi.to_device(I.target_hiddens(shape, wl, 0, nmax))
    ws = abi.Workspace(abi.mtp_workspace_bytes(head.cfg, nmax, cap))
    hout = torch.zeros((1, shape.hidden), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    amax = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    steps = max(args.steps, 3)

    def timed(n, mode, kind=None):
        def flush():
            abi.mtp_flush_pairs(head, kv, toks, hids, n, None, mode, 1, hout, logits, amax, ws, stream)
            abi.kv_rollback(kv, prefix, None, 0, stream)
        for _ in range(args.warmup):
            flush()
        torch.cuda.synchronize()
        if kind is not None:
            abi.mtp_timing_begin(kind, 64 * steps + 4)
        t = time.perf_counter()
        for i in range(steps):
            if kind is not None:
                abi.mtp_timing_pause(i % TIME_EVERY != 0)
            flush()
        torch.cuda.synchronize()
        el = (time.perf_counter() - t) / steps
        k = abi.mtp_timing_end() if kind is not None else None
        if int(kv.state[3].item()) != 0:
            raise RuntimeError("device error word set")
        return el, k

    curve = {}
    for n in sizes:
        t_last, _ = timed(n, abi.LAST)
        t_kv, _ = timed(n, abi.KV_ONLY)
        curve[n] = {"last_us": round(t_last * 1e6, 2), "kv_only_us": round(t_kv * 1e6, 2)}
        log(f"n={n}: LAST {t_last * 1e6:.1f} us, KV_ONLY {t_kv * 1e6:.1f} us")
    base = curve[sizes[0]]["last_us"] / sizes[0]
    for n in sizes:
        c = curve[n]
        c["cost_vs_n_steps"] = round(c["last_us"] / (n * base), 4)
        # LAST: every row's fc and q/k/v; the last row's attention (prefix + n keys), o, MLP and unembedding
        last_flops = 4 * shape.head_dim * shape.n_q_heads * (prefix + n) + flush_projection_flops(shape, n, 1)
        c["tflops_last"] = round(last_flops / (c["last_us"] * 1e-6) / 1e12, 2)
    # the largest flush's products, timed with events around their launches
    _, (proj_ms, proj_n) = timed(nmax, abi.LAST, abi.TIME_PROJECTION)
    timed_n = (steps + TIME_EVERY - 1) // TIME_EVERY
    proj_s = proj_ms / timed_n / 1e3
    gemm_flops = flush_projection_flops(shape, nmax, 1) - 2 * shape.vocab * shape.hidden
    t_big = curve[nmax]["last_us"] * 1e-6
    out = base_line(args, round(nmax / t_big, 1), "flushed pairs/s", t_big * 1e3, "bf16",
                    "synthetic (seeded N(0,0.02) weights of the Qwen3.5-27B-shaped head in bf16; uniform tokens, "
                    "N(0,1) bf16 hiddens; N(0,1) bf16 prefix K/V)",
                    {"workload": "flush_scaling_qwen35_27b_prefix4096", "hidden": shape.hidden,
                     "heads": f"{shape.n_q_heads}q/{shape.n_kv_heads}kv", "head_dim": shape.head_dim,
                     "intermediate": shape.intermediate, "vocab": shape.vocab, "prefix": prefix,
                     "pairs": sizes, "mode": "LAST (every row's K/V; last row's g, logits, argmax) and KV_ONLY"})
    out.update({
        "cost_curve": {str(n): curve[n] for n in sizes},
        "cost_curve_note": "cost_vs_n_steps = flush(n) / (n x flush(%d) / %d): below 1 means n positions cost "
                           "less than n separate steps" % (sizes[0], sizes[0]),
        "roofline": roofline("mfma", gemm_flops / proj_s / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", None,
                             kernel=f"the {nmax}-pair LAST flush's projections: fc and q/k/v over every row "
                                    "(MFMA products past 16 rows, GEMV passes below), o, gate/up and down for "
                                    "the last row (GEMV)",
                             flops_per_launch=round(gemm_flops / max(1, proj_n // timed_n)),
                             avg_us=round(proj_s * 1e6 / max(1, proj_n // timed_n), 2), launches=proj_n),
        "cpu_baseline": None,
    })
    return out


def cpu_flush(shape, storage, kp, vp, cap, prefix, toks, hids, seconds, max_flushes, cache_fp64=False):
    from mtp_draft_head_step_amd import inputs as I
    from oracle import head as OH
    from oracle.kvcache import DraftKV
    oh = OH.Head(shape, I.weight_values(shape, storage), cache_fp64=cache_fp64)
    tk = [int(t) for t in toks]
    hv = [I.decode(h, shape.act_dtype) for h in hids]
    K, V = I.decode(kp, shape.kv_dtype), I.decode(vp, shape.kv_dtype)
    def unit(_):
        okv = DraftKV(shape.n_kv_heads, cap, shape.head_dim, K, V, prefix)
        oh.flush(okv, tk, hv, OH.ALL, set_round_base=True)
    if cache_fp64:   # the large head: BLAS on every host thread, one flush
        flushes, el = timed_sample(unit, 0, 1)
        cores = cpu_threads()
    else:
        with single_thread_blas():
            flushes, el = timed_sample(unit, seconds, max_flushes)
        cores = 1
    return {"value": round(len(tk) * flushes / el, 4), "unit": "flushed pairs/s", "cores": cores, "kind": "oracle",
            "sample": f"{flushes} flush(es) of the same 256 pairs in ALL mode, numpy fp64"}


# ---------------------------------------------------------------------------
# sampled verification
# ---------------------------------------------------------------------------
VERIFY_POOL = 64


def run_verify(args):
    import numpy as np
    import torch

    from mtp_draft_head_step_amd import abi
    from mtp_draft_head_step_amd import inputs as I

    wl, N, V = I.WL_VERIFY, 4, 152064
    steps = args.steps
    top_k = args.top_k
    sp = abi.sampling(0.7, 1.1, top_k, 0.9, 0.05, 64)
    full = not (1 <= top_k <= 215)     # past the per-chunk candidates: the whole-vocabulary path
    t0 = time.time()
    rows = np.stack([I.logits_rows(wl, 5, r, N + 1, V, 4.0, spikes=3, spike=12.0)[0] for r in range(VERIFY_POOL)])
    drows = np.stack([I.logits_rows(wl, 6, r, N, V, 4.0)[0] for r in range(VERIFY_POOL)])
    t_rows, t_drows = abi.to_device(rows), abi.to_device(drows)
    ring0, st0 = I.history_ring(wl, None, 64, V)
    ring, ring_st = abi.to_device(ring0), abi.to_device(st0)
    # draft tokens: d_i drawn from q_i (history ++ d_<i) by the library's own
    # sampler (a verification of no drafts over the draft row) on a ring copy
    vws0 = abi.Workspace(abi.spec_verify_workspace_bytes(0, V))
    drafts = torch.zeros((VERIFY_POOL, N), dtype=torch.int32, device="cuda")
    du = abi.to_device(np.stack([I.uniforms(wl, r, N, stream=10) for r in range(VERIFY_POOL)]))
    tmp_c = torch.zeros(2, dtype=torch.int32, device="cuda")
    for r in range(VERIFY_POOL):
        rc, sc = ring.clone(), ring_st.clone()
        for i in range(N):
            abi.spec_verify(sp, 0, V, t_drows[r, i], None, None, rc, sc, du[r, i:i + 1], drafts[r, i:i + 1],
                            tmp_c, vws0)
    total = args.warmup + steps
    uni = abi.to_device(np.stack([I.uniforms(wl, (1, r), N + 1) for r in range(total)]))
    out_t = torch.zeros((total, N + 1), dtype=torch.int32, device="cuda")
    out_c = torch.zeros((total, 2), dtype=torch.int32, device="cuda")
    vws = abi.Workspace(abi.spec_verify_workspace_bytes(N, V))
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"verify inputs resident ({time.time() - t0:.1f}s): {VERIFY_POOL} rounds of logits, "
        f"{(rows.nbytes + drows.nbytes) >> 20} MiB")

    def one(r):
        p = r % VERIFY_POOL
        abi.spec_verify(sp, N, V, t_rows[p], t_drows[p], drafts[p], ring, ring_st, uni[r], out_t[r], out_c[r],
                        vws, stream)

    for r in range(args.warmup):
        one(r)
    torch.cuda.synchronize()
    abi.mtp_timing_begin(abi.TIME_VERIFY, steps + 4)
    t = time.perf_counter()
    for r in range(args.warmup, total):
        abi.mtp_timing_pause(r % TIME_EVERY != 0)
        one(r)
    torch.cuda.synchronize()
    el = time.perf_counter() - t
    ms, nl = abi.mtp_timing_end()
    counts = out_c[args.warmup:].cpu().numpy()
    if counts.min() < 0 or np.any(counts[:, 1] != counts[:, 0] + 1):
        raise RuntimeError("verification returned malformed counts")

    # greedy mode: temperature 0, 2 drafts, 3 target rows (1.82 MB) of the same pool
    gsp = abi.sampling(window=64)
    gws = abi.Workspace(abi.spec_verify_workspace_bytes(2, V))
    gring, gst = ring.clone(), ring_st.clone()

    def one_greedy(r):
        p = r % VERIFY_POOL
        abi.spec_verify(gsp, 2, V, t_rows[p], None, drafts[p], gring, gst, None, out_t[r % total],
                        out_c[r % total], gws, stream)
    g_steps = max(steps // 4, 100)
    for r in range(args.warmup):
        one_greedy(r)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for r in range(g_steps):
        one_greedy(r)
    torch.cuda.synchronize()
    g_el = time.perf_counter() - t
    g_bytes = 3 * V * 4 + 64 * 4
    calibrate_copy(args)
    # the timed first pass reads every row (the whole-vocabulary path also writes
    # the transformed rows back)
    chunk_bytes = (2 * N + 1) * V * 4 * (2 if full else 1) + 64 * 4
    avg = ms / nl / 1e3
    cpu = cpu_verify(rows, drows, ring0, st0, wl, N, args.cpu_seconds, total, top_k) if args.cpu_seconds > 0 \
        else None
    name = "verify_sampled_n4_v152064" if top_k == 40 else f"verify_sampled_n4_v152064_topk{top_k}"
    out = base_line(args, round(steps / el, 1), "verify rounds/s", el / steps * 1e3, "f32",
                    "synthetic (seeded N(0,4) fp32 target rows with 3 spikes of +12, N(0,4) draft rows, "
                    "64 resident rounds cycled, fresh uniforms per round)",
                    {"workload": name, "n_draft": N, "vocab": V, "temperature": 0.7,
                     "repeat_penalty": 1.1, "window": 64, "top_k": top_k, "top_p": 0.9, "min_p": 0.05})
    out.update({
        "us_per_round": round(el / steps * 1e6, 2),
        "round_gbs": round(chunk_bytes / (el / steps) / 1e9, 1),
        "mean_accepted": round(float(counts[:, 0].mean()), 4),
        "greedy": {"rows": 3, "drafts": 2, "rounds_per_s": round(g_steps / g_el, 1),
                   "us_per_round": round(g_el / g_steps * 1e6, 2),
                   "gbs": round(g_bytes / (g_el / g_steps) / 1e9, 1),
                   "hbm_frac": round(g_bytes / (g_el / g_steps) / 1e9 / HBM_PEAK_GBS, 4),
                   "note": "temperature 0 (argmax match), 3 target rows of the same pool, eager launches"},
        "roofline": roofline("hbm", chunk_bytes / avg / 1e9, HBM_PEAK_GBS, "GB/s", None,
                             kernel=("whole-vocabulary transform pass over the 9 rows (penalty, temperature, "
                                     "row maxima; transformed rows written back)" if full else
                                     "per-chunk top-k pass over the 9 rows (penalty, temperature, top-k above a floor, sorted)"),
                             bytes_per_launch=chunk_bytes, avg_us=round(avg * 1e6, 2), launches=nl),
        "cpu_baseline": with_host(cpu),
    })
    return out


def cpu_verify(rows, drows, ring0, st0, wl, N, seconds, max_rounds, top_k=40):
    import numpy as np

    from mtp_draft_head_step_amd import inputs as I
    from oracle import verify as OV
    sp = OV.Sampling(temperature=0.7, repeat_penalty=1.1, top_k=top_k, top_p=0.9, min_p=0.05, window=64)
    state = {"ring": np.array(ring0), "st": np.array(st0)}

    def unit(r):
        # the oracle draws its own drafts from q_i with the same seeded uniforms
        p = r % VERIFY_POOL
        ring, st = state["ring"], state["st"]
        du = I.uniforms(wl, p, N, stream=10)
        d = []
        for i in range(N):
            d.append(OV.sample(sp, drows[p, i], ring, st, float(du[i]), prefix=d))
        res = OV.verify(sp, rows[p], drows[p], d, ring, st, I.uniforms(wl, (1, r), N + 1))
        state["ring"], state["st"] = res["ring"], res["state"]
    n_rounds, el = timed_sample(unit, seconds, max_rounds)
    return {"value": round(n_rounds / el, 3), "unit": "verify rounds/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_rounds} rounds (draft draws + verification), numpy fp64 sort-based transforms"}


# ---------------------------------------------------------------------------
# depth sweep over a 32768-slot prefix
# ---------------------------------------------------------------------------
def committed_check(committed, expected):
    """The mean committed tokens per round against the closed form
    1 + sum_j prod_{i<j} p_i: a z-score over the rounds' own spread, passing
    within 4 standard errors."""
    import numpy as np
    c = np.asarray(committed, dtype=np.float64)
    R = len(c)
    se = float(c.std(ddof=1)) / np.sqrt(R) if R > 1 else float("nan")
    z = (float(c.mean()) - expected) / se if se > 0 else 0.0
    return {"rounds": R, "mean": round(float(c.mean()), 4), "std_err": round(se, 4), "z": round(z, 2),
            "within_4_se": bool(abs(z) <= 4.0)}


def run_depth(args, N, lm):
    import numpy as np
    import torch

    from mtp_draft_head_step_amd import abi
    from mtp_draft_head_step_amd import inputs as I

    ctx, S, policy = 32768, args.sessions, args.policy
    shape = I.TINY_BF16.with_dtypes(lm_head_dtype=I.I8G128 if lm == "i8g128" else I.BF16)
    wl, V, H = I.WL_DEPTH, shape.vocab, shape.hidden
    R = args.warmup + args.steps
    per_session = (R + S - 1) // S
    cap = ctx + per_session * (N + 1) + 64
    t0 = time.time()
    storage = I.head_weights(shape, wl)
    head = abi.Head(shape, storage)
    kp, vp = I.prefix_kv(shape, wl, ctx, cap)
    pool_hid = abi.to_device(np.stack([I.target_hiddens(shape, wl, r, N + 1) for r in range(POOL)]))
    first_tok = int(I.tokens_uniform(wl, 1, ctx + 2, V)[-1])
    first_hid = abi.to_device(I.target_hiddens(shape, wl, 1000, 1)[0])
    first_rows = torch.zeros((N + 1, H), dtype=torch.bfloat16, device="cuda")
    first_rows[0].copy_(first_hid)
    ws = abi.Workspace(abi.mtp_workspace_bytes(head.cfg, N + 1, cap))
    vws = abi.Workspace(abi.spec_verify_workspace_bytes(N, V))
    sp = abi.sampling(window=64)
    sessions = []
    for _ in range(S):
        iost = torch.zeros(4 + 2 + N + 1, dtype=torch.int32, device="cuda")  # {state | k, k+1, tokens}
        sessions.append({
            "iost": iost,
            "kv": abi.DraftKV(shape, cap, kp, vp, ctx, state=iost[0:4]),
            "io": iost[4:],
            "pend_t": torch.zeros(N + 1, dtype=torch.int32, device="cuda"),
            "pend_h": torch.zeros((N + 1, H), dtype=torch.bfloat16, device="cuda"),
            "n_dev": torch.zeros(1, dtype=torch.int32, device="cuda"),
            "d": torch.zeros(N, dtype=torch.int32, device="cuda"),
            "g": torch.zeros((N, H), dtype=torch.bfloat16, device="cuda"),
            "ring": torch.zeros(64, dtype=torch.int32, device="cuda"),
            "ring_st": torch.zeros(2, dtype=torch.int32, device="cuda"),
        })
    step_out = torch.zeros(H, dtype=torch.bfloat16, device="cuda")
    step_tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    log(f"{S} sessions of a {ctx}-slot KV resident ({time.time() - t0:.1f}s)")

    def reset():
        for s in sessions:
            s["kv"].state.copy_(torch.tensor([ctx, ctx, 0, 0], dtype=torch.int32))
            s["ring"].zero_()
            s["ring_st"].zero_()
            s["io"].zero_()
            s["io"][1] = 1
            s["io"][2] = first_tok
        torch.cuda.synchronize()

    base_rows = [I.logits_rows(wl, 5, r, N + 1, V, 3.0)[0] for r in range(POOL)]
    planted = torch.zeros((R, N + 1, V), dtype=torch.float32, device="cuda")
    k_of = [I.acceptance_draws(wl, r, N) for r in range(R)]
    prev_round = {}                                    # session -> its previous round

    def j0_of(k):
        return 0 if policy == "A" else min(k, N - 1)

    def pending_of(s):
        """The session's pending pairs.  Policy A: the previous verify's tokens
        (io[2:]), that round's target hiddens and the count io[1], as they stand.
        Policy B: pend_t / pend_h / n_dev, rebuilt on the device by
        mtp_repair_pending.  Round 0: the one initial pair."""
        ss = sessions[s]
        pr = prev_round.get(s)
        if pr is None:
            return ss["io"][2:], first_rows, ss["io"][1:2]
        if policy == "A":
            return ss["io"][2:], pool_hid[pr % POOL], ss["io"][1:2]
        return ss["pend_t"], ss["pend_h"], ss["n_dev"]

    def draft(s, st):
        ss = sessions[s]
        toks, hid, cnt = pending_of(s)
        abi.mtp_draft_chain(head, ss["kv"], toks, hid, N + 1, cnt, N, ss["d"], ss["g"], None, ws, st)

    def verify_and_rollback(s, r, st, report=None):
        ss = sessions[s]
        abi.spec_verify_rollback(sp, N, V, planted[r], None, ss["d"], ss["ring"], ss["ring_st"], None,
                                 ss["io"][2:], ss["io"][0:2], vws, ss["kv"], abi.TO_ROUND_BASE, policy == "B",
                                 report, st)
        if policy == "B":
            abi.mtp_repair_pending(ss["io"][2:], ss["io"][0:2], pool_hid[r % POOL], H, abi.MTP_BF16, N,
                                   ss["pend_t"], ss["pend_h"], ss["n_dev"], st)
        prev_round[s] = r

    # recording pass: the drafts decide where the acceptance is planted
    stream = torch.cuda.current_stream()
    reset()
    t0 = time.time()
    lens, committed = [], []
    for r in range(R):
        s = r % S
        before = int(sessions[s]["kv"].state[0].item())
        pr = prev_round.get(s)
        n_pend = 1 if pr is None else k_of[pr] + 1 - j0_of(k_of[pr])
        draft(s, stream)
        d = sessions[s]["d"].cpu().numpy()
        rows = base_rows[r % POOL].copy()
        I.plant_acceptance(rows, d.astype(np.int64), k_of[r])
        planted[r].copy_(torch.from_numpy(rows))
        verify_and_rollback(s, r, stream)
        k = int(sessions[s]["io"][0].item())
        if k != k_of[r]:
            raise RuntimeError(f"planted acceptance {k_of[r]} but verification accepted {k} in round {r}")
        lens.append((before, n_pend))
        committed.append(sessions[s]["io"][2:2 + k + 1].cpu().tolist())
    log(f"recording pass: {R} rounds in {time.time() - t0:.1f}s")

    # timed replay: the same device work, host sync per round overlapped
    reset()
    prev_round.clear()
    host = HostRows(POOL, 4 + 2 + N + 1)
    got = [None] * R

    def enqueue(r):
        s = r % S
        draft(s, stream)
        verify_and_rollback(s, r, stream, host.addr(r % POOL))   # the round's results to the host

    def consume(r):
        row = host.view[r % POOL]
        if int(row[3]) != 0:
            raise RuntimeError(f"device error word in round {r}")
        got[r] = row[6: 6 + int(row[5])].tolist()

    for r in range(args.warmup):
        enqueue(r)
        stream.synchronize()
        consume(r)
    abi.mtp_timing_begin(abi.TIME_ATTENTION, args.steps * N + 4)
    torch.cuda.synchronize()
    t = time.perf_counter()
    prev = None
    for r in range(args.warmup, R):
        abi.mtp_timing_pause(not (r % TIME_EVERY == 0 or r == args.warmup))
        enqueue(r)
        host.record(r % POOL, stream)
        if prev is not None:
            host.wait(prev % POOL)
            consume(prev)
        prev = r
    host.wait(prev % POOL)
    consume(prev)
    torch.cuda.synchronize()
    el = time.perf_counter() - t
    host.close()
    att_ms, att_n = abi.mtp_timing_end()
    if got != committed:
        raise RuntimeError("the timed replay committed a different stream than the recording pass")

    # chained draft steps alone, rotating sessions (their KV lengths restored after)
    n_steps = 8 * S
    st_before = [s["kv"].state.clone() for s in sessions]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n_steps):
        ss = sessions[i % S]
        abi.mtp_draft_step(head, ss["kv"], ss["d"][0:1], ss["g"][0], step_out, None, step_tok, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / n_steps
    for s, stb in zip(sessions, st_before):
        s["kv"].state.copy_(stb)
    calibrate_copy(args)

    att_bytes = 0                       # over the rounds whose attention launches were timed
    for r in range(args.warmup, R):
        if r % TIME_EVERY == 0 or r == args.warmup:
            before, n_pend = lens[r]
            att_bytes += sum(attention_bytes(shape, before + n_pend + i) for i in range(N))
    att_avg = att_ms / att_n / 1e3
    ks = np.array(k_of[args.warmup:])
    expected = 1.0 + sum(float(np.prod([0.8 * 0.85 ** i for i in range(j)])) for j in range(1, N + 1))
    committed_tok = int(sum(int(k) + 1 for k in ks))
    # the oracle runs one session in the same capacity: at most as many rounds as fit
    cpu_rounds_max = max(1, min(R, (cap - ctx - 64) // (N + 1)))
    cpu = cpu_depth(shape, storage, kp, vp, cap, ctx, N, policy, base_rows, args.cpu_seconds / len(
        str(args.depth).split(",")), cpu_rounds_max) if args.cpu_seconds > 0 else None
    out = base_line(args, round(N * args.steps / el, 2), "draft tokens/s", el / args.steps * 1e3, "bf16",
                    "synthetic (seeded N(0,0.02) tiny-head weights in bf16, N(0,1) bf16 prefix K/V, N(0,3) "
                    "target rows with planted greedy acceptance p_i = 0.8*0.85^i)",
                    {"workload": "depth_ctx32768", "hidden": H, "heads": "4q/2kv", "head_dim": 64,
                     "intermediate": shape.intermediate, "vocab": V, "draft_kv_context": ctx, "depth": N,
                     "lm_head": lm, "policy": policy, "sessions": S, "batch": 1, "temperature": 0.0})
    out.update({
        "rounds_per_s": round(args.steps / el, 2),
        "us_per_round": round(el / args.steps * 1e6, 2),
        "us_per_draft_step": round(step_us, 2),
        "committed_per_round": round(committed_tok / args.steps, 4),
        "committed_per_round_closed_form": round(expected, 4),
        "committed_check": committed_check(ks + 1, expected),
        "committed_tokens_per_s": round(committed_tok / el, 1),
        "roofline": roofline("hbm", att_bytes / (att_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s", None,
                             kernel="split-K attention over the 32768+ slot draft KV (2 kv heads, D 64, bf16)",
                             bytes_per_launch=round(att_bytes / att_n), avg_us=round(att_avg * 1e6, 2),
                             launches=att_n),
        "cpu_baseline": with_host(cpu),
    })
    return out


def run_depth_auto(args):
    """Rounds of the tiny bf16 head over a 32768-slot prefix whose depth is chosen
    every round by the library's depth controller (mtp_depth_ctl_*): it maximises
    committed tokens per unit of round time from the per-position acceptance it
    observes and a per-depth cost table.  Acceptance is planted with p_i = 0.8 *
    0.85^i per position, greedy, policy A; depth 0 is a plain-decode round (the
    pending pairs flushed KV_ONLY and one target row verified).  The cost table
    is seeded by timing 4 rounds at each depth, then every round reports its own
    GPU time (HIP events around its launches) plus --target-ms, a modelled target
    forward per round (no target model runs here; the pages' cost is the
    per-width forward cost, which the target's forward dominates).  One host
    synchronisation per round.  value = committed tokens over the controller's
    rounds / (their wall-clock time + rounds x target-ms)."""
    import numpy as np
    import torch

    from mtp_draft_head_step_amd import abi
    from mtp_draft_head_step_amd import inputs as I

    ctx, Dm = 32768, int(args.max_depth)
    shape = I.TINY_BF16
    wl, V, H = I.WL_DEPTH, shape.vocab, shape.hidden
    calib = 4
    R = (Dm + 1) * calib + args.warmup + args.steps
    cap = ctx + R * (Dm + 1) + 2 * (Dm + 1) + 64
    storage = I.head_weights(shape, wl)
    head = abi.Head(shape, storage)
    kp, vp = I.prefix_kv(shape, wl, ctx, cap)
    iost = torch.zeros(4 + 2 + Dm + 1, dtype=torch.int32, device="cuda")   # {state | k, k+1, tokens}
    kv = abi.DraftKV(shape, cap, kp, vp, ctx, state=iost[0:4])
    io = iost[4:]
    pool_hid = abi.to_device(np.stack([I.target_hiddens(shape, wl, r, Dm + 1) for r in range(POOL)]))
    base_rows = abi.to_device(np.stack([I.logits_rows(wl, 5, r, Dm + 1, V, 3.0)[0] for r in range(POOL)]))
    rows = torch.zeros((Dm + 1, V), dtype=torch.float32, device="cuda")
    first_hid = torch.zeros((Dm + 1, H), dtype=torch.bfloat16, device="cuda")
    first_hid[0].copy_(abi.to_device(I.target_hiddens(shape, wl, 1000, 1)[0]))
    d_buf = torch.zeros(Dm, dtype=torch.int32, device="cuda")
    g_buf = torch.zeros((Dm, H), dtype=torch.bfloat16, device="cuda")
    ring = torch.zeros(64, dtype=torch.int32, device="cuda")
    ring_st = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = abi.Workspace(abi.mtp_workspace_bytes(head.cfg, Dm + 1, cap))
    vws = abi.Workspace(abi.spec_verify_workspace_bytes(Dm, V))
    sp = abi.sampling(window=64)
    io[1] = 1
    io[2] = int(I.tokens_uniform(wl, 1, ctx + 2, V)[-1])
    host = torch.zeros(iost.numel(), dtype=torch.int32).pin_memory()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    state = {"hid": first_hid, "len": ctx}

    def round_(r, d):
        """Enqueue round r at depth d, wait for it; -> (k, GPU ms, kv length before, pending)."""
        k_plan = I.acceptance_draws(wl, (77, r), d) if d else 0
        before, n_pend = state["len"], int(host[5]) if r else 1
        e0.record(stream)
        if d:
            abi.mtp_draft_chain(head, kv, io[2:], state["hid"], Dm + 1, io[1:2], d, d_buf, g_buf, None, ws, stream)
        else:
            abi.mtp_flush_pairs(head, kv, io[2:], state["hid"], Dm + 1, io[1:2], abi.KV_ONLY, 1, None, None, None,
                                ws, stream)
        rows[: d + 1].copy_(base_rows[r % POOL][: d + 1])
        if d:
            I.plant_acceptance(rows, d_buf[:d].long(), k_plan)
        abi.spec_verify(sp, d, V, rows, None, d_buf, ring, ring_st, None, io[2:], io[0:2], vws, stream)
        if d:
            abi.kv_rollback(kv, abi.TO_ROUND_BASE, None, d, stream)
        e1.record(stream)
        host.copy_(iost, non_blocking=True)
        stream.synchronize()
        if int(host[3]) != 0:
            raise RuntimeError(f"device error word {int(host[3])} in round {r}")
        k = int(host[4])
        if k != k_plan:
            raise RuntimeError(f"planted acceptance {k_plan} but verification accepted {k} in round {r}")
        state["hid"] = pool_hid[r % POOL]
        state["len"] = int(host[0])
        return k, e0.elapsed_time(e1), before, n_pend

    # seed: 4 rounds at each depth
    tgt = float(args.target_ms)
    r = 0
    seed = []
    for d in range(Dm + 1):
        ts = []
        for _ in range(calib):
            ts.append(round_(r, d)[1])
            r += 1
        seed.append(float(np.median(ts)) + tgt)
    ctl = abi.DepthController(Dm, seed)
    for _ in range(args.warmup):
        d = ctl.next()
        k, ms, _, _ = round_(r, d)
        ctl.report(d, k, ms + tgt)
        r += 1
    hist = [0] * (Dm + 1)
    committed = 0
    att = []                                     # (before, pending, depth) of rounds with timed attention
    abi.mtp_timing_begin(abi.TIME_ATTENTION, args.steps * Dm + 4)
    t = time.perf_counter()
    for i in range(args.steps):
        d = ctl.next()
        timed = i % TIME_EVERY == 0
        abi.mtp_timing_pause(not timed)
        k, ms, before, n_pend = round_(r, d)
        ctl.report(d, k, ms + tgt)
        hist[d] += 1
        committed += k + 1
        if timed:
            att.append((before, n_pend, d))
        r += 1
    el = time.perf_counter() - t
    att_ms, att_n = abi.mtp_timing_end()
    choice, interval, cost = ctl.state()
    p = [0.8 * 0.85 ** i for i in range(Dm)]

    def exp_committed(n):
        tot, run = 1.0, 1.0
        for i in range(n):
            run *= p[i]
            tot += run
        return tot
    predicted = {str(n): round(exp_committed(n) / (seed[n] * 1e-3), 1) for n in range(Dm + 1)}   # seed includes tgt
    att_bytes = sum(attention_bytes(shape, b + n + i) for b, n, d in att for i in range(d))
    att_avg = att_ms / att_n / 1e3 if att_n else None
    cpu = cpu_depth_auto(shape, storage, kp, vp, cap, ctx, Dm, seed, tgt, args.cpu_seconds) \
        if args.cpu_seconds > 0 else None
    span = el + args.steps * tgt / 1e3
    out = base_line(args, round(committed / span, 2), "committed tokens/s", span / args.steps * 1e3, "bf16",
                    "synthetic (seeded N(0,0.02) tiny-head weights in bf16, N(0,1) bf16 prefix K/V, N(0,3) "
                    "target logits with planted acceptance p_i = 0.8*0.85^i)",
                    {"workload": "depth_auto_ctx32768", "hidden": H, "heads": f"{shape.n_q_heads}q/{shape.n_kv_heads}kv",
                     "head_dim": shape.head_dim, "vocab": V, "draft_kv_context": ctx, "max_depth": Dm,
                     "batch": 1, "temperature": 0.0, "policy": "A", "depth": "chosen per round by the controller",
                     "target_forward_ms_modelled": tgt})
    out.update({
        "depth_histogram": {str(n): hist[n] for n in range(Dm + 1) if hist[n]},
        "final_choice": choice, "probe_interval": interval,
        "seed_round_ms": [round(c, 4) for c in seed],
        "final_cost_ms": [round(c, 4) for c in cost],
        "fixed_depth_committed_per_gpu_s": predicted,
        "committed_per_round": round(committed / args.steps, 4),
        "measured_committed_per_s_without_target": round(committed / el, 2),
        "launch": "eager, one host sync per round (the controller needs each round's outcome)",
        "roofline": roofline("hbm", att_bytes / (att_ms / 1e3) / 1e9 if att_n else None, HBM_PEAK_GBS, "GB/s",
                             None, kernel="decode attention over the 32768-slot draft KV (chunk partials)",
                             avg_us=round(att_avg * 1e6, 2) if att_avg else None, launches=att_n),
        "cpu_baseline": with_host(cpu),
    })
    return out


def cpu_depth_auto(shape, storage, kp, vp, cap, ctx, Dm, seed, tgt, seconds):
    """The oracle as it stands on the same controller-driven workload: oracle
    rounds at the depth the oracle controller picks, its cost table seeded with
    the GPU's per-depth round times and fed the oracle's own round times (both
    plus the same modelled target forward)."""
    import numpy as np

    from mtp_draft_head_step_amd import inputs as I
    from oracle import depth as OD
    from oracle import head as OH
    from oracle import rounds as OR
    from oracle import verify as OV
    from oracle.kvcache import DraftKV
    wl, V = I.WL_DEPTH, shape.vocab
    oh = OH.Head(shape, I.weight_values(shape, storage))
    okv = DraftKV(shape.n_kv_heads, cap, shape.head_dim, I.decode(kp, shape.kv_dtype), I.decode(vp, shape.kv_dtype),
                  ctx)
    committed = [int(t) for t in I.tokens_uniform(wl, 1, ctx + 2, V)]
    hid0 = I.decode(I.target_hiddens(shape, wl, 1000, 1)[0], shape.act_dtype)
    st = OR.RoundState(oh, okv, [(committed[-1], hid0)], committed, window=64)
    ctl = OD.DepthController(Dm, seed)
    base = [I.logits_rows(wl, 5, r, Dm + 1, V, 3.0)[0] for r in range(POOL)]
    total = {"tokens": 0}

    def unit(r):
        d = ctl.next_depth()
        k_plan = I.acceptance_draws(wl, (77, r), d) if d else 0
        hid = I.decode(I.target_hiddens(shape, wl, r % POOL, Dm + 1), shape.act_dtype)
        t0 = time.perf_counter()
        if d:
            def fn(tokens, start):
                rows = base[r % POOL][: d + 1].copy()
                I.plant_acceptance(rows, np.asarray(tokens[1:], np.int64), k_plan)
                return rows, hid[: d + 1]
            k = OR.run_round(st, d, fn)["k"]
        else:
            oh.flush(okv, [t for t, _ in st.pending], [h for _, h in st.pending], OH.KV_ONLY, set_round_base=True)
            res = OV.verify(OV.Sampling(), base[r % POOL][:1], None, [], st.ring, st.ring_state)
            st.ring, st.ring_state = res["ring"], res["state"]
            st.pending = [(res["tokens"][0], hid[0])]
            st.committed.extend(res["tokens"])
            k = 0
        ctl.report(d, k, (time.perf_counter() - t0) * 1e3 + tgt)
        total["tokens"] += k + 1
    with single_thread_blas():
        n_rounds, el = timed_sample(unit, seconds, max(1, (cap - ctx - 64) // (Dm + 1) - 2))
    return {"value": round(total["tokens"] / (el + n_rounds * tgt / 1e3), 3), "unit": "committed tokens/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{n_rounds} controller-driven rounds of one session (oracle controller, planted acceptance) "
                      f"over the 32768-slot prefix, numpy fp64, one BLAS thread"}


def cpu_depth(shape, storage, kp, vp, cap, ctx, N, policy, base_rows, seconds, max_rounds):
    import numpy as np

    from mtp_draft_head_step_amd import inputs as I
    from oracle import head as OH
    from oracle import rounds as OR
    from oracle.kvcache import DraftKV
    wl = I.WL_DEPTH
    oh = OH.Head(shape, I.weight_values(shape, storage))
    okv = DraftKV(shape.n_kv_heads, cap, shape.head_dim, I.decode(kp, shape.kv_dtype), I.decode(vp, shape.kv_dtype),
                  ctx)
    committed = [int(t) for t in I.tokens_uniform(wl, 1, ctx + 2, shape.vocab)]
    hid0 = I.decode(I.target_hiddens(shape, wl, 1000, 1)[0], shape.act_dtype)
    st = OR.RoundState(oh, okv, [(committed[-1], hid0)], committed, window=64)
    def unit(r):
        k_r = I.acceptance_draws(wl, r, N)
        hid = I.decode(I.target_hiddens(shape, wl, r % POOL, N + 1), shape.act_dtype)

        def fn(tokens, start):
            rows = base_rows[r % POOL].copy()
            I.plant_acceptance(rows, np.asarray(tokens[1:], np.int64), k_r)
            return rows, hid
        OR.run_round(st, N, fn, policy=policy)
    with single_thread_blas():
        n_rounds, el = timed_sample(unit, seconds, max_rounds)
    return {"value": round(N * n_rounds / el, 3), "unit": "draft tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_rounds} rounds of one session at depth {N} (flush + chained steps + greedy "
                      f"verification + rollback over the 32768-slot prefix), numpy fp64, one BLAS thread"}


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (rounds, flushes or verify rounds)")
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="qwen35_27b_round",
                    choices=["qwen35_27b_round", "tiny_round", "flush256_prefix8192", "flush256_qwen35_27b",
                             "verify_sampled", "depth_ctx32768", "flush_scaling_qwen35_27b",
                             "depth_auto_ctx32768", "launch_floor", "batch_qwen35_27b"])
    ap.add_argument("--batch", type=int, default=4, help="batch_qwen35_27b: sessions per batched call (1..16)")
    ap.add_argument("--depth", default="4", help="depth_ctx32768: drafts per round (comma list: one line each)")
    ap.add_argument("--lm", default="bf16", choices=["bf16", "i8g128"],
                    help="qwen35_27b_round, depth_ctx32768: lm_head storage (int8 per (row, 128-column group) "
                         "with fp16 scales, or bf16)")
    ap.add_argument("--rows", default="1,2,3,4,6,8,12,16,24,32,48,64,96,128,192,256",
                    help="flush_scaling_qwen35_27b: pair counts of the flushes timed (comma list, 1..256)")
    ap.add_argument("--max-depth", type=int, default=8, help="depth_auto_ctx32768: deepest draft the controller may pick")
    ap.add_argument("--target-ms", type=float, default=2.0,
                    help="depth_auto_ctx32768: modelled target forward per round, added to each round's cost "
                         "(0 = the drafting machinery alone)")
    ap.add_argument("--policy", default="B", choices=["A", "B"], help="depth_ctx32768: KV policy")
    ap.add_argument("--sessions", type=int, default=32, help="depth_ctx32768: sessions rotated (1 = warm)")
    ap.add_argument("--top-k", type=int, default=40,
                    help="verify_sampled: top_k (0 = the whole vocabulary, served by the whole-vocabulary path)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of the oracle sample for cpu_baseline (0 = skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run three 1 GiB device-to-device copies (a plain copy kernel of known "
                         "size, to scale HBM traffic counters)")
    ap.add_argument("--graph", action="store_true",
                    help="qwen35_27b_round: replay rounds from HIP graphs only (no kernel timing in this mode)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed repeats of --steps steps; the line reports the median with min and max")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the MTP round is a batch-1 path on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    default_steps = {"qwen35_27b_round": 40, "tiny_round": 64, "flush256_prefix8192": 50, "flush256_qwen35_27b": 16,
                     "verify_sampled": 10000, "depth_ctx32768": 256, "flush_scaling_qwen35_27b": 16, "depth_auto_ctx32768": 600,
                     "launch_floor": 8, "batch_qwen35_27b": 40}
    if args.steps is None:
        args.steps = default_steps[args.workload]

    import torch  # noqa: F401  (the HIP runtime comes up before libmtp loads)

    from mtp_draft_head_step_amd import inputs as I
    if args.workload == "qwen35_27b_round":
        i8 = args.lm == "i8g128"
        shape = I.QWEN35_27B.with_dtypes(lm_head_dtype=I.I8G128) if i8 else I.QWEN35_27B
        lines = [run_greedy_rounds(args, shape, I.WL_QWEN, 4096, 2,
                                   "qwen35_27b_mtp_head_round" + ("_lm_i8g128" if i8 else ""),
                                   "synthetic (seeded N(0,0.02) weights of the Qwen3.5-27B MTP head shape"
                                   + ("; lm_head quantised int8 per (row, 128-column group), fp16 scales" if i8
                                      else "") + "; N(0,3) target logits, N(0,1) target hiddens)")]
    elif args.workload == "tiny_round":
        lines = [run_greedy_rounds(args, I.TINY_F32, I.WL_TINY, 128, 2, "tiny_f32_head_round",
                                   "synthetic (seeded N(0,0.02) tiny-head weights in fp32; N(0,3) target "
                                   "logits, N(0,1) target hiddens)", use_graphs=True)]
    elif args.workload == "flush256_prefix8192":
        lines = [run_flush(args)]
    elif args.workload == "flush256_qwen35_27b":
        lines = [run_flush(args, big=True)]
    elif args.workload == "verify_sampled":
        lines = [run_verify(args)]
    elif args.workload == "flush_scaling_qwen35_27b":
        lines = [run_flush_scaling(args)]
    elif args.workload == "depth_auto_ctx32768":
        lines = [run_depth_auto(args)]
    elif args.workload == "launch_floor":
        lines = [run_launch_floor(args)]
    elif args.workload == "batch_qwen35_27b":
        lines = [run_batch_rounds(args)]
    else:
        lines = [run_depth(args, int(d), args.lm) for d in str(args.depth).split(",")]
    for line in lines:
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
