"""GPU parity of greedy verification, rollback and whole rounds (policy A and B)
against the oracle, through the C ABI."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mtp_draft_head_step_amd import inputs as I
from oracle import head as OH
from oracle import rounds as R
from oracle import verify as OV
from oracle.kvcache import DraftKV
from tests.gpu_util import build, device_array, host, kv_pair

pytestmark = pytest.mark.gpu


def run_verify(sp, rows, drows, drafts, ring, ring_state, u=None):
    from mtp_draft_head_step_amd import abi
    n = len(drafts)
    v = rows.shape[1]
    ws = abi.Workspace(abi.spec_verify_workspace_bytes(n, v))
    t_ring = device_array(ring.astype(np.int32))
    t_st = device_array(ring_state.astype(np.int32))
    out_t = torch.full((n + 1,), -1, dtype=torch.int32, device="cuda")
    out_c = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    abi.spec_verify(sp, n, v, device_array(rows.astype(np.float32)),
                    None if drows is None else device_array(drows.astype(np.float32)),
                    device_array(np.asarray(drafts, np.int32)) if n else None, t_ring, t_st,
                    None if u is None else device_array(np.asarray(u, np.float32)), out_t, out_c, ws)
    torch.cuda.synchronize()
    k, c = host(out_c).tolist()
    return {"k": k, "count": c, "tokens": host(out_t)[: k + 1].tolist(), "ring": host(t_ring),
            "state": host(t_st)}


@pytest.mark.parametrize("vocab", [152064, 1000, 4097, 7])
@pytest.mark.parametrize("n", [0, 1, 2, 4, 8, 16])
@pytest.mark.parametrize("penalty", [1.0, 1.1])
def test_greedy_verify_parity(vocab, n, penalty):
    from mtp_draft_head_step_amd import abi
    rng = np.random.default_rng([vocab, n, int(penalty * 10)])
    window = 64
    for trial in range(3):
        rows = (rng.standard_normal((n + 1, vocab)) * 3).astype(np.float32)
        drafts = rng.integers(0, vocab, n)
        k_plant = int(rng.integers(0, n + 1))
        I.plant_acceptance(rows, drafts, k_plant, spike=20.0)
        # history holding some argmax tokens so the penalty can flip decisions
        ring = rng.integers(0, vocab, window).astype(np.int32)
        am = np.argmax(rows, axis=1)[:4]
        ring[: len(am)] = am
        st = np.array([int(rng.integers(0, window)), window], np.int32)
        sp_o = OV.Sampling(repeat_penalty=penalty, window=window)
        sp_g = abi.sampling(repeat_penalty=penalty, window=window)
        ref = OV.verify(sp_o, rows, None, list(drafts), ring, st)
        got = run_verify(sp_g, rows, None, drafts, ring, st)
        assert got["k"] == ref["k"] and got["count"] == ref["k"] + 1
        assert got["tokens"] == ref["tokens"]
        assert np.array_equal(got["ring"], ref["ring"]) and np.array_equal(got["state"], ref["state"])


def test_greedy_ties_pick_lowest_id():
    from mtp_draft_head_step_amd import abi
    rows = np.zeros((3, 9000), np.float32)
    rows[1, [17, 8001, 4096]] = 5.0
    got = run_verify(abi.sampling(), rows, None, [0, 17], np.zeros(8, np.int32), np.array([0, 0], np.int32))
    assert got["k"] == 2 and got["tokens"] == [0, 17, 0]
    assert got["state"].tolist() == [3, 3] and got["ring"][:3].tolist() == [0, 17, 0]


def test_rollback_device_semantics():
    from mtp_draft_head_step_amd import abi
    shape = I.TINY_F32
    gkv, _ = kv_pair(shape, 90, 10, 64)
    kbytes = host(gkv.k).copy()
    gkv.state.copy_(torch.tensor([14, 11, 0, 0], dtype=torch.int32))
    abi.kv_rollback(gkv, abi.TO_ROUND_BASE)                      # policy A
    torch.cuda.synchronize()
    assert host(gkv.state).tolist() == [11, 11, 0, 0]
    gkv.state.copy_(torch.tensor([14, 11, 0, 0], dtype=torch.int32))
    for k, want in ((0, 11), (1, 12), (2, 13), (3, 13), (7, 13)):  # policy B, N = 3
        gkv.state.copy_(torch.tensor([14, 11, 0, 0], dtype=torch.int32))
        abi.kv_rollback(gkv, abi.TO_ROUND_BASE, torch.tensor([k], dtype=torch.int32, device="cuda"), 3)
        torch.cuda.synchronize()
        assert host(gkv.state)[0] == want
    abi.kv_rollback(gkv, 5)
    torch.cuda.synchronize()
    assert host(gkv.state).tolist()[:1] == [5]
    abi.kv_rollback(gkv, 9)                                       # beyond the length
    torch.cuda.synchronize()
    assert host(gkv.state).tolist() == [5, 11, 0, abi.DEV_ROLLBACK]
    assert np.array_equal(host(gkv.k), kbytes)                    # no K/V byte moved


# ---------------------------------------------------------------- whole rounds
SHAPE = I.HeadShape(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=256, vocab=96)
L0, CAP = 8, 256


def successor_storage(seed=22):
    """fp32 storage of the head whose greedy draft is (token + 1) mod V."""
    st = I.head_weights(SHAPE, seed)
    h = SHAPE.hidden
    st["fc"] = np.zeros((h, 2 * h), np.float32)
    st["fc"][:, :h] = np.eye(h)
    st["o_proj"] = np.zeros_like(st["o_proj"])
    st["down_proj"] = np.zeros_like(st["down_proj"])
    for n in I.NORM_TENSORS:
        st[n] = np.ones_like(st[n])
    e = np.random.default_rng(seed).standard_normal((SHAPE.vocab, h)).astype(np.float32)
    st["embed"] = e
    st["lm_head"] = np.ascontiguousarray(np.roll(e, 1, axis=0))
    return st


def gpu_session(st_storage, tgt, n_draft):
    from mtp_draft_head_step_amd import abi
    gh = abi.Head(SHAPE, st_storage)
    oh = OH.Head(SHAPE, I.weight_values(SHAPE, st_storage))
    kp, vp = I.prefix_kv(SHAPE, 9, L0, CAP)
    gkv = abi.DraftKV(SHAPE, CAP, kp, vp, L0)
    okv = DraftKV(SHAPE.n_kv_heads, CAP, SHAPE.head_dim, kp, vp, L0)
    committed = [int(t) for t in np.random.default_rng(5).integers(0, SHAPE.vocab, L0 + 2)]
    pending = [(committed[s + 1], tgt.hidden_state(committed[s], s)) for s in range(L0, L0 + 1)]
    return gh, oh, gkv, okv, committed, pending


@pytest.mark.parametrize("policy", ["A", "B"])
@pytest.mark.parametrize("n_draft", [1, 2, 3])
@pytest.mark.parametrize("headkind", ["random", "successor"])
def test_rounds_match_oracle_and_classic(policy, n_draft, headkind):
    """GPU rounds (flush LAST with the device count from the previous verify,
    chained steps, greedy verify, rollback) commit the oracle's stream, which is
    classic greedy decoding; the draft KV lengths follow the oracle exactly."""
    from mtp_draft_head_step_amd import abi
    storage = I.head_weights(SHAPE, 21) if headkind == "random" else successor_storage()
    tgt = I.ToyTarget(31, SHAPE.vocab, SHAPE.hidden, follow=0.8 if headkind == "successor" else 0.0)
    gh, oh, gkv, okv, committed, pending = gpu_session(storage, tgt, n_draft)
    ost = R.RoundState(oh, okv, pending, committed, window=16)
    start = list(committed)
    N = n_draft
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, N + 1, CAP))
    vws = abi.Workspace(abi.spec_verify_workspace_bytes(N, SHAPE.vocab))
    ring = torch.zeros(16, dtype=torch.int32, device="cuda")
    ring_st = torch.zeros(2, dtype=torch.int32, device="cuda")
    d_buf = torch.zeros(N, dtype=torch.int32, device="cuda")
    g_buf = torch.zeros((N, SHAPE.hidden), dtype=torch.float32, device="cuda")
    out_t = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    out_c = torch.zeros(2, dtype=torch.int32, device="cuda")
    pend_t = device_array(np.array([t for t, _ in pending] + [0] * N, np.int32))
    pend_h = device_array(np.concatenate([np.stack([h for _, h in pending]),
                                          np.zeros((N, SHAPE.hidden), np.float32)]))
    n_dev = torch.tensor([len(pending)], dtype=torch.int32, device="cuda")
    gpu_committed = list(committed)
    ks = []
    diverged = False
    for rnd in range(12):
        abi.mtp_flush_pairs(gh, gkv, pend_t, pend_h, N + 1, n_dev, abi.LAST, 1, g_buf[0], None, d_buf[0:1], ws)
        for i in range(1, N):
            abi.mtp_draft_step(gh, gkv, d_buf[i - 1:i], g_buf[i - 1], g_buf[i], None, d_buf[i:i + 1], ws)
        drafts = host(d_buf).tolist()
        c = len(gpu_committed) - 1
        rows, hid_rows = tgt.forward([gpu_committed[-1]] + drafts, c)
        abi.spec_verify(abi.sampling(window=16), N, SHAPE.vocab, device_array(rows), None, d_buf,
                        ring, ring_st, None, out_t, out_c, vws)
        abi.kv_rollback(gkv, abi.TO_ROUND_BASE, out_c[0:1] if policy == "B" else None, N)
        k = int(host(out_c)[0])
        toks = host(out_t)[: k + 1].tolist()
        j0 = 0 if policy == "A" else min(k, N - 1)
        pend_t[: k + 1 - j0] = out_t[j0:k + 1]
        pend_h[: k + 1 - j0] = device_array(hid_rows[j0:k + 1])
        n_dev.fill_(k + 1 - j0)
        gpu_committed += toks
        ks.append(k)
        # oracle round on the same inputs
        out = R.run_round(ost, N, lambda tk, s: tgt.forward(tk, s), policy=policy)
        diverged = diverged or out["drafts"] != drafts   # a draft near tie: both valid
        st = host(gkv.state)
        assert st[3] == 0
        if not diverged:
            assert st[0] == ost.kv.len, (rnd, st, ost.kv.len)
    assert gpu_committed == ost.committed
    assert gpu_committed == R.classic_greedy(lambda tk, s: tgt.forward(tk, s), start, len(gpu_committed) - len(start))
    if headkind == "successor":
        assert max(ks) == N and min(ks) == 0


@pytest.mark.parametrize("headkind", ["random", "successor"])
def test_rounds_with_changing_depth_match_classic(headkind):
    """Rounds whose depth changes every round, plain decode (depth 0) included,
    as the depth controller drives them: the flush takes the host bound of the
    deepest round and the previous round's device count; a depth-0 round flushes
    its pending pairs KV_ONLY and verifies one target row.  The GPU commits the
    oracle's stream, which is classic greedy decoding, with the same draft KV
    lengths (policy A)."""
    from mtp_draft_head_step_amd import abi
    storage = I.head_weights(SHAPE, 23) if headkind == "random" else successor_storage()
    tgt = I.ToyTarget(33, SHAPE.vocab, SHAPE.hidden, follow=0.8 if headkind == "successor" else 0.0)
    Dm = 3
    gh, oh, gkv, okv, committed, pending = gpu_session(storage, tgt, Dm)
    ost = R.RoundState(oh, okv, pending, committed, window=16)
    start = list(committed)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, Dm + 1, CAP))
    vws = abi.Workspace(abi.spec_verify_workspace_bytes(Dm, SHAPE.vocab))
    ring = torch.zeros(16, dtype=torch.int32, device="cuda")
    ring_st = torch.zeros(2, dtype=torch.int32, device="cuda")
    d_buf = torch.zeros(Dm, dtype=torch.int32, device="cuda")
    g_buf = torch.zeros((Dm, SHAPE.hidden), dtype=torch.float32, device="cuda")
    out_t = torch.zeros(Dm + 1, dtype=torch.int32, device="cuda")
    out_c = torch.zeros(2, dtype=torch.int32, device="cuda")
    pend_t = device_array(np.array([t for t, _ in pending] + [0] * Dm, np.int32))
    pend_h = device_array(np.concatenate([np.stack([h for _, h in pending]),
                                          np.zeros((Dm, SHAPE.hidden), np.float32)]))
    n_dev = torch.tensor([len(pending)], dtype=torch.int32, device="cuda")
    gpu_committed = list(committed)
    depths = [2, 0, 3, 1, 0, 3, 3, 1, 2, 0, 0, 3, 2, 1]
    diverged = False
    for rnd, d in enumerate(depths):
        c = len(gpu_committed) - 1
        if d:
            abi.mtp_draft_chain(gh, gkv, pend_t, pend_h, Dm + 1, n_dev, d, d_buf, g_buf, None, ws)
            drafts = host(d_buf)[:d].tolist()
        else:
            abi.mtp_flush_pairs(gh, gkv, pend_t, pend_h, Dm + 1, n_dev, abi.KV_ONLY, 1, None, None, None, ws)
            drafts = []
        rows, hid_rows = tgt.forward([gpu_committed[-1]] + drafts, c)
        abi.spec_verify(abi.sampling(window=16), d, SHAPE.vocab, device_array(rows), None, d_buf,
                        ring, ring_st, None, out_t, out_c, vws)
        if d:
            abi.kv_rollback(gkv, abi.TO_ROUND_BASE, None, d)
        k = int(host(out_c)[0])
        toks = host(out_t)[: k + 1].tolist()
        pend_t[: k + 1] = out_t[: k + 1]
        pend_h[: k + 1] = device_array(hid_rows[: k + 1])
        n_dev.fill_(k + 1)
        gpu_committed += toks
        # the oracle on the same inputs
        if d:
            out = R.run_round(ost, d, lambda tk, s: tgt.forward(tk, s), policy="A")
            diverged = diverged or out["drafts"] != drafts
        else:
            oh.flush(okv, [t for t, _ in ost.pending], [h for _, h in ost.pending], OH.KV_ONLY,
                     set_round_base=True)
            orow, ohid = tgt.forward([ost.committed[-1]], len(ost.committed) - 1)
            res = OV.verify(OV.Sampling(window=16), orow, None, [], ost.ring, ost.ring_state)
            ost.ring, ost.ring_state = res["ring"], res["state"]
            ost.pending = [(res["tokens"][0], ohid[0])]
            ost.committed.extend(res["tokens"])
        st = host(gkv.state)
        assert st[3] == 0
        if not diverged:
            assert st[0] == ost.kv.len, (rnd, d, st, ost.kv.len)
    assert gpu_committed == ost.committed
    assert gpu_committed == R.classic_greedy(lambda tk, s: tgt.forward(tk, s), start, len(gpu_committed) - len(start))


GRAPH_SHAPES = {
    "tiny_bf16": I.TINY_BF16,
    "h2048_bf16": I.HeadShape(hidden=2048, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=4096,
                              vocab=8192).with_dtypes(weight_dtype=I.BF16, act_dtype=I.BF16, kv_dtype=I.BF16,
                                                      lm_head_dtype=I.BF16),
}


def _round_session(shape, wl, n_draft, pool, cap):
    from mtp_draft_head_step_amd import abi
    st = I.head_weights(shape, wl)
    gh = abi.Head(shape, st)
    kp, vp = I.prefix_kv(shape, wl, 64, cap)
    kv = abi.DraftKV(shape, cap, kp, vp, 64)
    V, H, N = shape.vocab, shape.hidden, n_draft
    dt = torch.bfloat16 if shape.act_dtype == I.BF16 else torch.float32
    s = {
        "gh": gh, "kv": kv,
        "logits": device_array(np.stack([I.logits_rows(wl, 5, r, N + 1, V, 3.0)[0] for r in range(pool)])),
        "hid": device_array(np.stack([I.target_hiddens(shape, wl, r, N + 1) for r in range(pool)])),
        "io": torch.zeros(2 + N + 1, dtype=torch.int32, device="cuda"),
        "d": torch.zeros(N, dtype=torch.int32, device="cuda"),
        "g": torch.zeros((N, H), dtype=dt, device="cuda"),
        "ring": torch.zeros(64, dtype=torch.int32, device="cuda"),
        "ring_st": torch.zeros(2, dtype=torch.int32, device="cuda"),
        "ws": abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, N + 1, cap)),
        "vws": abi.Workspace(abi.spec_verify_workspace_bytes(N, V)),
    }
    s["io"][1] = 1
    s["io"][2] = 5
    return s


def _enqueue(s, r, N, pool, stream):
    from mtp_draft_head_step_amd import abi
    io, d, g = s["io"], s["d"], s["g"]
    abi.mtp_flush_pairs(s["gh"], s["kv"], io[2:], s["hid"][(r - 1) % pool], N + 1, io[1:2], abi.LAST, 1,
                        g[0], None, d[0:1], s["ws"], stream)
    for i in range(1, N):
        abi.mtp_draft_step(s["gh"], s["kv"], d[i - 1:i], g[i - 1], g[i], None, d[i:i + 1], s["ws"], stream)
    abi.spec_verify(abi.sampling(window=64), N, s["gh"].shape.vocab, s["logits"][r % pool], None, d,
                    s["ring"], s["ring_st"], None, io[2:], io[0:2], s["vws"], stream)
    abi.kv_rollback(s["kv"], abi.TO_ROUND_BASE, None, N, stream)


@pytest.mark.parametrize("n_draft", [2, 3])
@pytest.mark.parametrize("shape_name", ["tiny_bf16", "h2048_bf16"])
def test_graph_replayed_rounds_equal_eager(n_draft, shape_name):
    """Rounds captured once into graphs and replayed many times (with eager work
    and host syncs between replays) commit the same tokens and leave the same
    draft KV as the same rounds launched eagerly.  The hidden-2048 head runs its
    flushes on the matrix cores (the weight-streaming fc product with the fused
    split reduce and row norm, 64 x 64 tiles for q/k/v)."""
    shape = GRAPH_SHAPES[shape_name]
    pool, rounds, cap = 4, 12, 512
    eager = _round_session(shape, 55, n_draft, pool, cap)
    graph = _round_session(shape, 55, n_draft, pool, cap)
    stream = torch.cuda.current_stream()
    ref_tokens = []
    for r in range(rounds):
        _enqueue(eager, r, n_draft, pool, stream)
        torch.cuda.synchronize()
        io = host(eager["io"])
        ref_tokens.append(io[2:2 + io[1]].tolist())
    # capture one graph per pool slot, after one eager round on the graph session
    _enqueue(graph, 0, n_draft, pool, stream)
    torch.cuda.synchronize()
    got = [host(graph["io"])[2:2 + host(graph["io"])[1]].tolist()]
    cs = torch.cuda.Stream()
    graphs = {}
    for p in range(1, pool + 1):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cs):
            _enqueue(graph, p, n_draft, pool, torch.cuda.current_stream())
        graphs[p % pool] = gr
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 16, device="cuda")
    for r in range(1, rounds):
        graphs[r % pool].replay()
        scratch.add_(1.0)                     # unrelated eager work between replays
        torch.cuda.synchronize()
        io = host(graph["io"])
        got.append(io[2:2 + io[1]].tolist())
    assert got == ref_tokens
    assert host(graph["kv"].state).tolist() == host(eager["kv"].state).tolist()
    n = int(host(eager["kv"].state)[0])
    assert torch.equal(graph["kv"].k[:, :n], eager["kv"].k[:, :n])
    assert torch.equal(graph["kv"].v[:, :n], eager["kv"].v[:, :n])
