#!/usr/bin/env python3
"""MTP round throughput on one MI355X.

Workload: the Qwen3.5-27B-shaped MTP head (H=5120, 24/4 heads, head_dim 256,
SwiGLU 17408, vocab 152064 borrowed lm_head), bf16 weights and activations with
fp32 accumulation, batch 1, draft KV context 4096, 2 drafts per round
(block_size 3), temperature 0, weights N(0, 0.02) seeded (synthetic: no
checkpoint).  One bench step is one MTP round, the whole hot path:
  flush of the completed pairs (LAST) -> 1 chained draft step -> greedy verify of
  the 3 target rows -> draft-KV rollback (policy A) -> one host sync reading the
  accepted count, committed tokens and the KV state.
Target logits rows (N(0, 3)) and target hiddens (N(0, 1)) are synthetic inputs
drawn per round from a pool of 8 resident rounds.

Every pointer and count of a round is device-resident, so the host enqueues
round r + 1 before it waits for round r: the round's host synchronisation
(reading k, the committed tokens and the KV error word) overlaps the next
round's GPU work.  --graph replays each round from a HIP graph instead.

Prints ONE JSON line.  value = draft tokens/s (2 per round); rounds/s is given
beside it.  roofline = the unembedding GEMV (the dominant kernel), timed with HIP
events around each of its launches inside the timed region.  cpu_baseline = the
fp64 numpy oracle running one round of the same workload on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
N_DRAFT = 2
CTX = 4096
POOL = 8


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_bytes(shape, ctx_len, with_logits=False):
    """Algorithmic HBM bytes of one draft-head step at KV length ctx_len (the new
    slot included): every weight once, one embedding row, the KV read and the new
    K/V row written, the hidden in/out, plus logits if they are written."""
    H, D, hkv, V = shape.hidden, shape.head_dim, shape.n_kv_heads, shape.vocab
    wb = 2 if shape.weight_dtype == "bf16" else 4
    kvb = 2 if shape.kv_dtype == "bf16" else 4
    ab = 2 if shape.act_dtype == "bf16" else 4
    head = shape.head_param_count() * wb
    lm = V * H * (1 if shape.lm_head_dtype == "i8g128" else wb)
    if shape.lm_head_dtype == "i8g128":
        lm += V * (H // 128) * 2
    kv = 2 * hkv * D * kvb * ctx_len
    return head + lm + H * wb + kv + 2 * H * ab + (V * 4 if with_logits else 0)


def unembed_bytes(shape):
    """Algorithmic bytes of one unembedding launch: the lm_head, the fp32 input
    vector, the final-norm weight (logits are not written in the timed rounds)."""
    H, V = shape.hidden, shape.vocab
    wb = 2 if shape.lm_head_dtype == "bf16" else (1 if shape.lm_head_dtype == "i8g128" else 4)
    extra = V * (H // 128) * 2 if shape.lm_head_dtype == "i8g128" else 0
    return V * H * wb + extra + H * 4 + H * 2


def gemv_source_digest():
    h = hashlib.sha256()
    for f in ("gemv.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "mtp_draft_head_step_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per unembedding launch from the committed rocprofv3 PMC summary,
    or None if there is none or the kernel source changed since it was taken."""
    p = os.path.join(ROOT, "profiles", "unembed_qwen35_27b_traffic.json")
    try:
        with open(p) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("gemv_source_digest") != gemv_source_digest():
        return None
    return d.get("bytes_per_launch")


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--cpu-rounds", type=int, default=1, help="oracle rounds for cpu_baseline (0 = skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run three 1 GiB device-to-device copies (a plain copy kernel of known "
                         "size, to scale HBM traffic counters)")
    ap.add_argument("--graph", action="store_true",
                    help="replay rounds from HIP graphs (no unembedding timing in this mode)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the MTP round is a batch-1 path on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mtp_draft_head_step_amd import abi
    from mtp_draft_head_step_amd import inputs as I

    shape, wl, N = I.QWEN35_27B, I.WL_QWEN, N_DRAFT
    V, H = shape.vocab, shape.hidden
    t0 = time.time()
    storage = I.head_weights(shape, wl)
    log(f"weights generated in {time.time() - t0:.1f}s")
    head = abi.Head(shape, storage)
    cap = CTX + 1 + (args.warmup + args.steps + 4) * (N + 1) + 64
    kp, vp = I.prefix_kv(shape, wl, CTX, cap)
    kv = abi.DraftKV(shape, cap, kp, vp, CTX)
    pool_logits = np.stack([I.logits_rows(wl, 5, r, N + 1, V, 3.0)[0] for r in range(POOL)])
    pool_hid = np.stack([I.target_hiddens(shape, wl, r, N + 1) for r in range(POOL)])
    first_tok = I.tokens_uniform(wl, 0, N + 1, V)
    first_hid = I.target_hiddens(shape, wl, 1000, N + 1)
    ring0, ring_st0 = I.history_ring(wl, None, 64, V)
    dev = "cuda"
    t_logits = abi.to_device(pool_logits)
    t_hid = abi.to_device(pool_hid)
    t_tok0 = abi.to_device(first_tok)
    t_hid0 = abi.to_device(first_hid)
    ring = abi.to_device(ring0)
    ring_st = abi.to_device(ring_st0)
    io = torch.zeros(2 + N + 1, dtype=torch.int32, device=dev)      # {k, k+1, tokens...}
    d_buf = torch.zeros(N, dtype=torch.int32, device=dev)
    g_buf = torch.zeros((N, H), dtype=torch.bfloat16, device=dev)
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
    io[2:] = t_tok0
    t_hid[POOL - 1].copy_(t_hid0)
    width = 2 + N + 1 + 4
    host = torch.zeros((POOL, width), dtype=torch.int32).pin_memory()
    totals = {"committed": 0, "accepted": 0}

    def enqueue_round(r, st):
        prev = (r - 1) % POOL
        abi.mtp_flush_pairs(head, kv, io[2:], t_hid[prev], N + 1, io[1:2], abi.LAST, 1,
                            g_buf[0], None, d_buf[0:1], ws, st)
        for i in range(1, N):
            abi.mtp_draft_step(head, kv, d_buf[i - 1:i], g_buf[i - 1], g_buf[i], None, d_buf[i:i + 1], ws, st)
        abi.spec_verify(sp, N, V, t_logits[r % POOL], None, d_buf, ring, ring_st, None, io[2:], io[0:2], vws, st)
        abi.kv_rollback(kv, abi.TO_ROUND_BASE, None, N, st)
        # the round's results for the host: k, k+1, tokens and the KV state words
        host[r % POOL, : 2 + N + 1].copy_(io, non_blocking=True)
        host[r % POOL, 2 + N + 1:].copy_(kv.state, non_blocking=True)

    def consume(r):
        row = host[r % POOL]
        if int(row[2 + N + 1 + 3]) != 0:
            raise RuntimeError(f"device error word {int(row[2 + N + 1 + 3])} in round {r}")
        totals["committed"] += int(row[1])
        totals["accepted"] += int(row[0])

    for r in range(args.warmup):                       # eager rounds
        enqueue_round(r, stream)
        stream.synchronize()
        consume(r)
    log(f"warmup {args.warmup} rounds done")

    graphs = None
    if args.graph:
        # one graph per pool slot (the unembedding timing is not available for
        # captured launches, so the roofline is left null in this mode)
        cap_stream = torch.cuda.Stream()
        graphs = {}
        for p_ in range(POOL):
            r = args.warmup + p_
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap_stream):
                enqueue_round(r, torch.cuda.current_stream())
            graphs[r % POOL] = g
        torch.cuda.synchronize()
        log("captured %d round graphs" % POOL)
    else:
        abi.mtp_timing_begin(args.steps * N + 4)

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    done = [torch.cuda.Event(), torch.cuda.Event()]
    prev = None
    for r in range(args.warmup, args.warmup + args.steps):
        if graphs is not None:
            graphs[r % POOL].replay()
        else:
            enqueue_round(r, stream)
        done[r % 2].record(stream)
        if prev is not None:                          # the one host sync per round,
            done[prev % 2].synchronize()              # overlapped with the next round
            consume(prev)
        prev = r
    done[prev % 2].synchronize()
    consume(prev)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    lm_ms, lm_n = (0.0, 0) if graphs is not None else abi.mtp_timing_end()
    log(f"timed {args.steps} rounds in {elapsed * 1e3:.1f} ms; unembedding {lm_n} launches")
    state = totals

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    rounds_s = args.steps / elapsed
    ms_step = elapsed / args.steps * 1e3
    lm_avg_s = lm_ms / lm_n / 1e3 if lm_n else None
    ub = unembed_bytes(shape)
    achieved = ub / lm_avg_s / 1e9 if lm_avg_s else None
    round_bytes = N * step_bytes(shape, CTX + 2) + (N + 1) * V * 4
    traffic = measured_traffic()

    cpu = None
    if args.cpu_rounds > 0:
        cpu = cpu_baseline(shape, storage, kp, vp, cap, pool_logits, pool_hid, first_tok, first_hid,
                           ring0, ring_st0, args.cpu_rounds)

    out = {
        "metric": "MTP draft tokens/sec + verify rounds/sec at batch 1 (GB/s vs HBM peak)",
        "value": round(N * rounds_s, 2),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights of the Qwen3.5-27B MTP head shape; N(0,3) target logits, N(0,1) target hiddens)",
        "config": {"workload": "qwen35_27b_mtp_head_round", "hidden": H, "heads": "24q/4kv",
                   "head_dim": 256, "intermediate": shape.intermediate, "vocab": V,
                   "draft_kv_context": CTX, "drafts_per_round": N, "block_size": N + 1,
                   "temperature": 0.0, "batch": 1, "policy": "A"},
        "rounds_per_s": round(rounds_s, 2),
        "round_gbs": round(round_bytes / (elapsed / args.steps) / 1e9, 1),
        "round_hbm_frac": round(round_bytes / (elapsed / args.steps) / 1e9 / HBM_PEAK_GBS, 4),
        "committed_per_round": round(state["committed"] / (args.warmup + args.steps), 4),
        "launch": ("hip graph per round" if args.graph else "eager") +
                  ", host sync per round overlapped with the next round",
        "roofline": None if achieved is None else {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "unembedding GEMV (lm_head 152064x5120 bf16)",
            "bytes_per_launch": ub, "avg_us": round(lm_avg_s * 1e6, 2), "launches": lm_n},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(shape, storage, kp, vp, cap, pool_logits, pool_hid, first_tok, first_hid, ring0,
                 ring_st0, rounds):
    """The oracle as it stands, on the host: `rounds` rounds of the same workload."""
    import numpy as np

    from mtp_draft_head_step_amd import inputs as I
    from oracle import head as OH
    from oracle import rounds as OR
    from oracle.kvcache import DraftKV
    t0 = time.time()
    vals = I.weight_values(shape, storage)
    oh = OH.Head(shape, vals)
    okv = DraftKV(shape.n_kv_heads, cap, shape.head_dim, I.decode(kp, "bf16"), I.decode(vp, "bf16"), CTX)
    pending = [(int(first_tok[0]), I.decode(first_hid[0], "bf16"))]
    committed = [0] * (CTX + 2)
    st = OR.RoundState(oh, okv, pending, committed, ring0, ring_st0, window=64)
    log(f"oracle inputs decoded in {time.time() - t0:.1f}s")

    def target_fn(toks, start):
        r = target_fn.r
        return pool_logits[r % POOL], I.decode(pool_hid[r % POOL], "bf16")
    t1 = time.perf_counter()
    for r in range(rounds):
        target_fn.r = r
        OR.run_round(st, N_DRAFT, target_fn, policy="A")
    el = time.perf_counter() - t1
    log(f"oracle {rounds} round(s) in {el:.1f}s")
    return {"value": round(N_DRAFT * rounds / el, 4), "unit": "draft tokens/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": f"{rounds} round(s) of the same workload (flush + 1 chained step + greedy verify + "
                      f"rollback at draft KV context {CTX}), numpy fp64"}


if __name__ == "__main__":
    main()
