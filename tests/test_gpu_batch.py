"""GPU parity of B > 1 independent sessions with ragged acceptance through the
batched C ABI (mtp_draft_chain_batch, spec_verify_batch, kv_rollback_batch,
mtp_repair_pending_batch) against the B-session oracle loop.

Every session starts at its own prefix length, has its own pending pairs,
history ring and target rows, and accepts its own planted number of drafts each
round (drawn per session and round with p_i = 0.8 * 0.85^i), so the sessions'
lengths drift apart and the next round's flush takes a different number of
pairs per session.  Each round, every session is compared with the oracle:
draft logits and hiddens (the oracle follows the GPU's drafts through near
ties), k, the committed tokens, the pending pairs, the KV length and round base,
and every appended K/V entry per head and slot."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mtp_draft_head_step_amd import inputs as I
from oracle import batch as OB
from oracle import head as OH
from oracle import rounds as R
from oracle import verify as OV
from oracle.kvcache import DraftKV
from tests.gpu_util import argmax_ok, assert_vectors, device_array, host, rel_err, tol_of

pytestmark = pytest.mark.gpu

H2048 = I.HeadShape(hidden=2048, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=4096,
                    vocab=8192).with_dtypes(weight_dtype=I.BF16, act_dtype=I.BF16, kv_dtype=I.BF16,
                                            lm_head_dtype=I.BF16)


def _dt(shape):
    return torch.bfloat16 if shape.act_dtype == I.BF16 else torch.float32


def batch_session(shape, wl, prefixes, cap, gh=None, oh=None):
    """GPU BatchKV and oracle sessions with prefix lengths ``prefixes``."""
    from mtp_draft_head_step_amd import abi
    if gh is None:
        st = I.head_weights(shape, wl)
        gh = abi.Head(shape, st)
        oh = OH.Head(shape, I.weight_values(shape, st))
    B = len(prefixes)
    ks, vs, states, hid0s = [], [], [], []
    for b, p in enumerate(prefixes):
        kp, vp = I.prefix_kv(shape, wl + 100 * b, p, cap)
        ks.append(kp)
        vs.append(vp)
        okv = DraftKV(shape.n_kv_heads, cap, shape.head_dim, I.decode(kp, shape.kv_dtype),
                      I.decode(vp, shape.kv_dtype), p)
        committed = [int(t) for t in I.tokens_uniform(wl, (1, b), p + 2, shape.vocab)]
        hid0 = I.target_hiddens(shape, wl, (1000, b), 1)[0]
        hid0s.append(hid0)
        states.append(R.RoundState(oh, okv, [(committed[-1], I.decode(hid0, shape.act_dtype))], committed,
                                   window=64))
    gkv = abi.BatchKV(shape, B, cap, np.stack(ks), np.stack(vs), prefixes)
    return gh, oh, gkv, states, hid0s


def run_batch_rounds(shape, gh, gkv, states, hid0s, N, targets, n_rounds, policy, check=True):
    """Rounds of every session launched as one batch; each round compared with
    the oracle session by session.  ``targets(rnd, b, drafts_b)`` -> (target
    logits [N+1, V] fp32, target hiddens [N+1, H] act dtype).  Returns the ks."""
    from mtp_draft_head_step_amd import abi
    B, H, V = len(states), shape.hidden, shape.vocab
    tol = tol_of(shape)
    i32 = dict(dtype=torch.int32, device="cuda")
    dt = _dt(shape)
    ws = abi.Workspace(abi.mtp_batch_workspace_bytes(gh.cfg, B, N + 1, gkv.capacity))
    vws = abi.Workspace(B * abi.spec_verify_workspace_bytes(N, V))
    ring, ring_st = torch.zeros((B, 64), **i32), torch.zeros((B, 2), **i32)
    d_buf = torch.zeros((B, N), **i32)
    g_buf = torch.zeros((B, N, H), dtype=dt, device="cuda")
    l_buf = torch.zeros((B, N, V), dtype=torch.float32, device="cuda")
    out_t, out_c = torch.zeros((B, N + 1), **i32), torch.zeros((B, 2), **i32)
    pend_t = torch.zeros((B, N + 1), **i32)
    pend_h = torch.zeros((B, N + 1, H), dtype=dt, device="cuda")
    pend_c = torch.ones(B, **i32)
    tgt_h = torch.zeros((B, N + 1, H), dtype=dt, device="cuda")
    for b, st in enumerate(states):
        pend_t[b, 0] = st.committed[-1]
        pend_h[b, 0] = device_array(hid0s[b])
    out_c[:, 1] = 1                              # policy A reads the counts from out_counts[:, 1]
    gpu_committed = [list(st.committed) for st in states]
    all_ks = []
    for rnd in range(n_rounds):
        base = host(gkv.state)[:, 0].copy()
        if policy == "A":
            n_dev, stride = out_c[:, 1:], 2
        else:
            n_dev, stride = pend_c, 1
        abi.mtp_draft_chain_batch(gh, gkv, B, pend_t, pend_h, N + 1, n_dev, stride, N, d_buf, g_buf, l_buf, ws)
        torch.cuda.synchronize()
        drafts = host(d_buf).tolist()
        rows = np.zeros((B, N + 1, V), np.float32)
        hids = []
        for b in range(B):
            rows[b], hb = targets(rnd, b, drafts[b])
            hids.append(hb)
        tgt_h.copy_(device_array(np.stack(hids)))
        abi.spec_verify_batch(abi.sampling(window=64), B, N, V, device_array(rows), None, d_buf, ring, ring_st,
                              None, out_t, out_c, vws)
        torch.cuda.synchronize()
        appended = host(gkv.state)[:, 0].copy()
        abi.kv_rollback_batch(gkv, B, abi.TO_ROUND_BASE, out_c if policy == "B" else None, N)
        if policy == "B":
            abi.mtp_repair_pending_batch(B, out_t, out_c, tgt_h, H, abi.config_of(shape).act_dtype, N, pend_t,
                                         pend_h, pend_c)
        else:
            pend_t.copy_(out_t)
            pend_h.copy_(tgt_h)
        torch.cuda.synchronize()
        ks = host(out_c)[:, 0].tolist()
        all_ks.append(ks)
        st_now = host(gkv.state)
        lgs, gs = host(l_buf), host(g_buf)
        outs = OB.run_batch_round(states, N, [(lambda tk, s, r=rows[b], h=hids[b]: (r, I.decode(h, shape.act_dtype)))
                                              for b in range(B)], policy=policy, forced_drafts=drafts)
        for b in range(B):
            k = ks[b]
            toks = host(out_t)[b, : k + 1].tolist()
            gpu_committed[b] += toks
            o = outs[b]
            assert o["k"] == k and o["tokens"] == toks, (rnd, b, o["k"], k)
            j0 = 0 if policy == "A" else min(k, N - 1)
            if policy == "B":
                assert int(host(pend_c)[b]) == k + 1 - j0
            assert host(pend_t)[b, : k + 1 - j0].tolist() == toks[j0:]
            assert st_now[b, 3] == 0
            assert st_now[b, 0] == states[b].kv.len and st_now[b, 1] == states[b].kv.base, (rnd, b)
            if not check:
                continue
            for i in range(N):
                ref = o["draft_logits"][i]
                assert rel_err(lgs[b, i], ref) <= tol, (rnd, b, i, rel_err(lgs[b, i], ref))
                assert rel_err(gs[b, i], o["draft_g"][i]) <= tol, (rnd, b, i)
                assert argmax_ok(drafts[b][i], ref, lgs[b, i])[0], (rnd, b, i)
            lo, hi = int(base[b]), int(appended[b])
            assert_vectors(host(gkv.k)[b, :, lo:hi], states[b].kv.K[:, lo:hi], tol, f"K round {rnd} session {b}")
            assert_vectors(host(gkv.v)[b, :, lo:hi], states[b].kv.V[:, lo:hi], tol, f"V round {rnd} session {b}")
    for b, st in enumerate(states):
        assert gpu_committed[b] == st.committed
    return all_ks


def planted_targets(shape, wl, N):
    def targets(rnd, b, drafts_b):
        k = I.acceptance_draws(wl, (rnd, b), N)
        rows = I.logits_rows(wl, 5, (rnd, b), N + 1, shape.vocab, 3.0)[0]
        I.plant_acceptance(rows, np.asarray(drafts_b, np.int64), k)
        return rows, I.target_hiddens(shape, wl, (rnd, b, 7), N + 1)
    return targets


CASES = {
    # (shape, sessions' prefix lengths, drafts, policy): the GEMV passes (up to
    # 16 flattened rows), the bf16 few-row passes, the matrix-core flush of a
    # small head (24 rows) and the weight-streaming products (hidden 2048)
    "tiny_f32_b4_A": (I.TINY_F32, [128, 40, 300, 7], 2, "A"),
    "tiny_f32_b4_B": (I.TINY_F32, [128, 40, 300, 7], 2, "B"),
    "tiny_bf16_b3_A": (I.TINY_BF16, [64, 65, 500], 3, "A"),
    "tiny_bf16_b6_A": (I.TINY_BF16, [10, 20, 30, 40, 50, 60], 3, "A"),
    # the last-row products at the largest batch, and with per-session pending
    # counts (policy B: each session's last row at its own index)
    "tiny_bf16_b16_A": (I.TINY_BF16, [5 + 19 * i for i in range(16)], 2, "A"),
    "tiny_bf16_b5_B": (I.TINY_BF16, [64, 7, 200, 33, 120], 3, "B"),
    # nine sessions: the unembedding in launches of four, four and one
    "tiny_f32_b9_A": (I.TINY_F32, [128, 40, 300, 7, 90, 11, 64, 200, 33], 2, "A"),
    "h2048_b2_B": (H2048, [333, 77], 2, "B"),
    # six sessions of a large-vocabulary head: the unembedding as one product
    "h2048_b6_A": (H2048, [333, 77, 120, 9, 250, 64], 2, "A"),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", list(CASES))
def test_batch_ragged_rounds(case):
    shape, prefixes, N, policy = CASES[case]
    wl = 120 + len(prefixes)
    cap = max(prefixes) + 12 * (N + 1) + 8
    gh, oh, gkv, states, hid0s = batch_session(shape, wl, prefixes, cap)
    ks = run_batch_rounds(shape, gh, gkv, states, hid0s, N, planted_targets(shape, wl, N), 12, policy)
    assert sum(len(set(k)) > 1 for k in ks) >= 3          # ragged acceptance within rounds


def test_batch_of_one_equals_single_session_chain():
    """mtp_draft_chain_batch with one session runs exactly mtp_draft_chain."""
    from mtp_draft_head_step_amd import abi
    shape = I.TINY_BF16
    st = I.head_weights(shape, 130)
    gh = abi.Head(shape, st)
    kp, vp = I.prefix_kv(shape, 130, 90, 256)
    kv1 = abi.DraftKV(shape, 256, kp, vp, 90)
    kvb = abi.BatchKV(shape, 1, 256, kp[None], vp[None], [90])
    N = 3
    toks = device_array(I.tokens_uniform(130, 4, N + 1, shape.vocab))
    hids = device_array(I.target_hiddens(shape, 130, 4, N + 1))
    n_dev = torch.tensor([2], dtype=torch.int32, device="cuda")
    outs = []
    for kv, batched in ((kv1, False), (kvb, True)):
        d = torch.full((N,), -1, dtype=torch.int32, device="cuda")
        g = torch.zeros((N, shape.hidden), dtype=torch.bfloat16, device="cuda")
        lg = torch.zeros((N, shape.vocab), dtype=torch.float32, device="cuda")
        if batched:
            ws = abi.Workspace(abi.mtp_batch_workspace_bytes(gh.cfg, 1, N + 1, 256))
            abi.mtp_draft_chain_batch(gh, kv, 1, toks, hids, N + 1, n_dev, 1, N, d, g, lg, ws)
        else:
            ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, N + 1, 256))
            abi.mtp_draft_chain(gh, kv, toks, hids, N + 1, n_dev, N, d, g, lg, ws)
        torch.cuda.synchronize()
        outs.append((d, g, lg))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert torch.equal(kv1.state, kvb.state[0]) and torch.equal(kv1.k, kvb.k[0]) and torch.equal(kv1.v, kvb.v[0])


@pytest.mark.parametrize("sampled", [False, True])
def test_verify_batch_equals_per_session(sampled):
    """spec_verify_batch over 4 sessions gives, bit for bit, each session's
    spec_verify (greedy with a penalty; sampled with the verification workload's
    settings, coverage-style draft rows)."""
    from mtp_draft_head_step_amd import abi
    B, N, V = 4, 3, 20000
    rng = np.random.default_rng(77)
    rows = (rng.standard_normal((B, N + 1, V)) * 3).astype(np.float32)
    drows = (rows[:, :N] + 0.5 * rng.standard_normal((B, N, V))).astype(np.float32)
    rings = rng.integers(0, V, (B, 64)).astype(np.int32)
    rst = np.stack([np.array([int(rng.integers(0, 64)), 64], np.int32) for _ in range(B)])
    u = rng.random((B, N + 1)).astype(np.float32)
    if sampled:
        sp = abi.sampling(0.7, 1.1, 40, 0.9, 0.05, 64)
        spo = OV.Sampling(temperature=0.7, repeat_penalty=1.1, top_k=40, top_p=0.9, min_p=0.05, window=64)
        d = np.array([[OV.sample(spo, drows[b, i], rings[b], rst[b], rng.random()) for i in range(N)]
                      for b in range(B)], np.int32)
    else:
        sp = abi.sampling(repeat_penalty=1.1, window=64)
        d = np.argmax(rows[:, :N], axis=2).astype(np.int32)
        d[1, 1] = (d[1, 1] + 1) % V                                # ragged: session 1 rejects at 1
        d[2, 0] = (d[2, 0] + 1) % V
    i32 = dict(dtype=torch.int32, device="cuda")
    ring_b, st_b = device_array(rings), device_array(rst)
    ot, oc = torch.full((B, N + 1), -1, **i32), torch.full((B, 2), -1, **i32)
    ws = abi.Workspace(B * abi.spec_verify_workspace_bytes(N, V))
    abi.spec_verify_batch(sp, B, N, V, device_array(rows), device_array(drows) if sampled else None,
                          device_array(d), ring_b, st_b, device_array(u) if sampled else None, ot, oc, ws)
    torch.cuda.synchronize()
    for b in range(B):
        ring1, st1 = device_array(rings[b]), device_array(rst[b])
        ot1, oc1 = torch.full((N + 1,), -1, **i32), torch.full((2,), -1, **i32)
        ws1 = abi.Workspace(abi.spec_verify_workspace_bytes(N, V))
        abi.spec_verify(sp, N, V, device_array(rows[b]), device_array(drows[b]) if sampled else None,
                        device_array(d[b]), ring1, st1, device_array(u[b]) if sampled else None, ot1, oc1, ws1)
        torch.cuda.synchronize()
        assert torch.equal(oc[b], oc1) and torch.equal(ot[b, : int(oc1[1])], ot1[: int(oc1[1])])
        assert torch.equal(ring_b[b], ring1) and torch.equal(st_b[b], st1)
    if not sampled:
        want = [OV.verify(OV.Sampling(repeat_penalty=1.1, window=64), rows[b], None, list(d[b]), rings[b],
                          rst[b])["k"] for b in range(B)]
        assert host(oc)[:, 0].tolist() == want and len(set(want)) > 1      # ragged


@pytest.mark.parametrize("shape", [I.TINY_F32, I.TINY_BF16], ids=["f32", "bf16"])
def test_batch_session_errors_are_isolated(shape):
    """A session whose pending count is 0 (or whose cache is full) gets its own
    error word; the other sessions of the batch proceed and match the oracle
    (bf16: o, the MLP and the unembedding as products over the gathered last
    rows, whose hidden copy must skip the failed sessions)."""
    from mtp_draft_head_step_amd import abi
    wl, N = 140, 2
    prefixes = [50, 60, 246]                     # session 2's cache is full: its flush cannot append
    cap = 246
    gh, oh, gkv, states, hid0s = batch_session(shape, wl, prefixes, cap)
    B, H, V = 3, shape.hidden, shape.vocab
    i32 = dict(dtype=torch.int32, device="cuda")
    ws = abi.Workspace(abi.mtp_batch_workspace_bytes(gh.cfg, B, N + 1, cap))
    pend_t = torch.zeros((B, N + 1), **i32)
    pend_h = torch.zeros((B, N + 1, H), dtype=_dt(shape), device="cuda")
    for b in range(B):
        pend_t[b, 0] = states[b].committed[-1]
        pend_h[b, 0] = device_array(hid0s[b])
    counts = torch.tensor([1, 0, 1], **i32)      # session 1 has nothing pending: a count error
    d = torch.full((B, N), -1, **i32)
    g = torch.zeros((B, N, H), dtype=_dt(shape), device="cuda")
    lg = torch.zeros((B, N, V), dtype=torch.float32, device="cuda")
    abi.mtp_draft_chain_batch(gh, gkv, B, pend_t, pend_h, N + 1, counts, 1, N, d, g, lg, ws)
    torch.cuda.synchronize()
    st = host(gkv.state)
    assert st[1].tolist() == [60, 60, 0, abi.DEV_COUNT]
    assert st[2].tolist() == [246, 246, 0, abi.DEV_CAPACITY]
    assert st[0].tolist() == [50 + 1 + N - 1, 51, 0, 0]
    assert np.all(host(d)[1:] == -1) and np.all(host(g)[1:] == 0)
    # session 0 equals the oracle's drafting of its pending pair
    o = states[0].head.flush(states[0].kv, [states[0].committed[-1]], [I.decode(hid0s[0], shape.act_dtype)],
                             OH.LAST, set_round_base=True)
    assert rel_err(host(lg)[0, 0], o["logits"]) <= tol_of(shape)
    assert rel_err(host(g)[0, 0], o["g"][-1]) <= tol_of(shape)
    assert argmax_ok(int(host(d)[0, 0]), o["logits"], host(lg)[0, 0])[0]
