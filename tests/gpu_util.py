"""Helpers shared by the GPU parity tests: build the same seeded head for the HIP
path and the oracle, move results back, and apply the parity tolerances.

Tolerances: fp32 heads max|gpu - ref| <= 1e-4 * max|ref| per row or vector;
bf16 heads 2e-2 * max|ref| (the activation and KV roundings to bf16 plus fp32
accumulation order).  Integer results (tokens, counts, lengths) are exact.
"""
import numpy as np

from mtp_draft_head_step_amd import inputs as I

F32_TOL = 1e-4
BF16_TOL = 2e-2


def tol_of(shape):
    return BF16_TOL if shape.weight_dtype == I.BF16 or shape.act_dtype == I.BF16 or shape.kv_dtype == I.BF16 else F32_TOL


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


def assert_vectors(gpu, ref, tol, what=""):
    """The tolerance per vector along the last axis: for every vector (a K or V
    entry of one head at one slot, a row of g or of logits),
    max|gpu - ref| <= tol * max|ref| of that vector."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.max(np.abs(g - r), axis=-1)
    scale = np.maximum(np.max(np.abs(r), axis=-1), 1e-30)
    bad = err > tol * scale
    if bad.any():
        first = np.argwhere(bad)[0].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} vector(s) past {tol:g} of their scale, worst "
                             f"{float(np.max(err / scale)):.3g}, first at {first}")


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def device_array(arr):
    from mtp_draft_head_step_amd import abi
    return abi.to_device(np.ascontiguousarray(arr))


def build(shape, wl):
    """(storage dict, GPU head, oracle head)."""
    from mtp_draft_head_step_amd import abi
    from oracle import head as OH
    st = I.head_weights(shape, wl)
    gh = abi.Head(shape, st)
    oh = OH.Head(shape, I.weight_values(shape, st))
    return st, gh, oh


def kv_pair(shape, wl, prefix, capacity):
    """A GPU DraftKV and an oracle DraftKV holding the same synthetic prefix."""
    from mtp_draft_head_step_amd import abi
    from oracle.kvcache import DraftKV
    kp, vp = I.prefix_kv(shape, wl, prefix, capacity)
    g = abi.DraftKV(shape, capacity, kp, vp, prefix)
    o = DraftKV(shape.n_kv_heads, capacity, shape.head_dim,
                I.decode(kp, shape.kv_dtype), I.decode(vp, shape.kv_dtype), prefix)
    return g, o


def argmax_ok(gpu_tok, ref_logits, gpu_logits):
    """The GPU argmax equals the oracle's, or the oracle's top-two margin is within
    twice the largest logit difference (a near tie, where both are correct)."""
    ref_tok = int(np.argmax(ref_logits))
    if int(gpu_tok) == ref_tok:
        return True, False
    bound = 2.0 * np.max(np.abs(np.asarray(gpu_logits, np.float64) - ref_logits))
    return bool(ref_logits[ref_tok] - ref_logits[int(gpu_tok)] <= bound), True


def compare_rounds(gh, oh, gkv, okv, shape, committed, hid0, n_draft, targets, n_rounds, policy="A",
                   window=64):
    """Greedy rounds launched as the benchmark launches them -- mtp_draft_chain
    over the pending pairs with their device count, spec_verify of the N + 1
    target rows, kv_rollback, and under policy B the device re-pairing -- next to
    the oracle's rounds on the same inputs, compared round by round: every draft
    step's logits and hidden output, the drafts (the oracle follows the GPU's
    drafts; where they differ from its argmax its top-two margin must lie within
    the logit tolerance), k, the committed tokens, the pending pairs, the KV
    lengths and every appended K/V entry per head and slot.

    ``targets(rnd, drafts)`` -> (target logits fp32 [N+1, V], target hiddens
    [N+1, H] in the activation dtype) for the round.  Returns (ks, near_ties)."""
    import torch
    from mtp_draft_head_step_amd import abi
    from oracle import rounds as R
    N, H, V = n_draft, shape.hidden, shape.vocab
    tol = tol_of(shape)
    i32 = dict(dtype=torch.int32, device="cuda")
    adt = torch.bfloat16 if shape.act_dtype == I.BF16 else torch.float32
    ost = R.RoundState(oh, okv, [(int(committed[-1]), I.decode(hid0, shape.act_dtype))],
                       [int(t) for t in committed], window=window)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, N + 1, gkv.capacity))
    vws = abi.Workspace(abi.spec_verify_workspace_bytes(N, V))
    ring, ring_st = torch.zeros(window, **i32), torch.zeros(2, **i32)
    d_buf = torch.zeros(N, **i32)
    g_buf = torch.zeros((N, H), dtype=adt, device="cuda")
    l_buf = torch.zeros((N, V), dtype=torch.float32, device="cuda")
    out_t, out_c = torch.zeros(N + 1, **i32), torch.zeros(2, **i32)
    pend_t = torch.zeros(N + 1, **i32)
    pend_t[0] = int(committed[-1])
    pend_h = torch.zeros((N + 1, H), dtype=adt, device="cuda")
    pend_h[0] = device_array(hid0)
    n_dev = torch.ones(1, **i32)
    tgt_h = torch.zeros((N + 1, H), dtype=adt, device="cuda")
    gpu_committed = [int(t) for t in committed]
    ks, near_ties = [], 0
    for rnd in range(n_rounds):
        base = int(host(gkv.state)[0])
        abi.mtp_draft_chain(gh, gkv, pend_t, pend_h, N + 1, n_dev, N, d_buf, g_buf, l_buf, ws)
        torch.cuda.synchronize()
        drafts = host(d_buf).tolist()
        rows, hid_st = targets(rnd, drafts)
        tgt_h.copy_(device_array(hid_st))
        abi.spec_verify(abi.sampling(window=window), N, V, device_array(rows), None, d_buf, ring, ring_st,
                        None, out_t, out_c, vws)
        torch.cuda.synchronize()
        appended = int(host(gkv.state)[0])
        abi.kv_rollback(gkv, abi.TO_ROUND_BASE, out_c[0:1] if policy == "B" else None, N)
        if policy == "B":
            abi.mtp_repair_pending(out_t, out_c, tgt_h, H, abi.config_of(shape).act_dtype, N, pend_t, pend_h,
                                   n_dev)
        else:
            pend_t.copy_(out_t)
            pend_h.copy_(tgt_h)
            n_dev.copy_(out_c[1:2])
        torch.cuda.synchronize()
        k = int(host(out_c)[0])
        toks = host(out_t)[: k + 1].tolist()
        gpu_committed += toks
        ks.append(k)
        j0 = 0 if policy == "A" else min(k, N - 1)
        assert int(host(n_dev)[0]) == k + 1 - j0
        assert host(pend_t)[: k + 1 - j0].tolist() == toks[j0:]
        out = R.run_round(ost, N, lambda tk, s: (rows, I.decode(hid_st, shape.act_dtype)), policy=policy,
                          forced_drafts=drafts)
        lgs, gs = host(l_buf), host(g_buf)
        for i in range(N):
            ref = out["draft_logits"][i]
            assert rel_err(lgs[i], ref) <= tol, (rnd, i, rel_err(lgs[i], ref))
            assert rel_err(gs[i], out["draft_g"][i]) <= tol, (rnd, i)
            ok, near = argmax_ok(drafts[i], ref, lgs[i])
            assert ok, (rnd, i)
            near_ties += near
        assert out["k"] == k and out["tokens"] == toks, (rnd, out["k"], k)
        st_now = host(gkv.state)
        assert st_now[3] == 0
        assert st_now[0] == ost.kv.len and st_now[1] == ost.kv.base, (rnd, st_now, ost.kv.len, ost.kv.base)
        assert_vectors(host(gkv.k)[:, base:appended], ost.kv.K[:, base:appended], tol, f"K round {rnd}")
        assert_vectors(host(gkv.v)[:, base:appended], ost.kv.V[:, base:appended], tol, f"V round {rnd}")
    assert gpu_committed == ost.committed
    return ks, near_ties
