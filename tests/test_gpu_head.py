"""GPU parity of the draft-head step and the pending-pair flush against the
oracle, through the C ABI (tiny fp32 head, tiny bf16 head)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mtp_draft_head_step_amd import inputs as I
from oracle import head as OH
from tests.gpu_util import argmax_ok, assert_vectors, build, device_array, host, kv_pair, rel_err, tol_of

pytestmark = pytest.mark.gpu

SHAPES = {"tiny_f32": I.TINY_F32, "tiny_bf16": I.TINY_BF16}


def act_dtype(shape):
    return torch.bfloat16 if shape.act_dtype == I.BF16 else torch.float32


def check_kv(gkv, okv, shape, lo, hi, tol):
    """Every K and V entry of slots [lo, hi), per head and slot."""
    assert_vectors(host(gkv.k)[:, lo:hi], okv.K[:, lo:hi], tol, "K")
    assert_vectors(host(gkv.v)[:, lo:hi], okv.V[:, lo:hi], tol, "V")


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("prefix", [0, 1, 100, 1000])
def test_step_parity(name, prefix):
    from mtp_draft_head_step_amd import abi
    shape = SHAPES[name]
    tol = tol_of(shape)
    wl = 40 + prefix
    _, gh, oh = build(shape, wl)
    cap = 1536
    gkv, okv = kv_pair(shape, wl, prefix, cap)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, 1, cap))
    tok = int(I.tokens_uniform(wl, 0, 1, shape.vocab)[0])
    hid = I.target_hiddens(shape, wl, 0, 1)
    t_tok = torch.tensor([tok], dtype=torch.int32, device="cuda")
    t_hid = device_array(hid)
    hout = torch.empty(shape.hidden, dtype=act_dtype(shape), device="cuda")
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    abi.mtp_draft_step(gh, gkv, t_tok, t_hid, hout, logits, amax, ws)
    torch.cuda.synchronize()
    ref = oh.step(okv, tok, I.decode(hid[0], shape.act_dtype))
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol, rel_err(lg, ref["logits"])
    assert rel_err(host(hout), ref["g"][0]) <= tol
    ok, _ = argmax_ok(int(host(amax)[0]), ref["logits"], lg)
    assert ok
    assert int(host(amax)[0]) == int(np.argmax(lg))          # the fused argmax of its own logits
    st = host(gkv.state)
    assert st[0] == prefix + 1 and st[3] == 0
    check_kv(gkv, okv, shape, 0, prefix + 1, tol)


@pytest.mark.parametrize("name", list(SHAPES))
def test_chained_steps(name):
    """Three chained steps: each feeds its own argmax and hidden output (on the
    device, no host round trip).  The oracle is teacher-forced: step i takes the
    GPU's token and its hidden output of step i - 1 (decoded from the activation
    dtype), so every step is held at the flat tolerance; the appended K/V of
    every step is compared per head and slot."""
    from mtp_draft_head_step_amd import abi
    shape = SHAPES[name]
    tol = tol_of(shape)
    wl = 60
    _, gh, oh = build(shape, wl)
    cap = 512
    gkv, okv = kv_pair(shape, wl, 200, cap)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, 1, cap))
    tok = torch.tensor([5], dtype=torch.int32, device="cuda")
    hid = I.target_hiddens(shape, wl, 0, 1)
    h_in = device_array(hid)[0]
    toks = [torch.empty(1, dtype=torch.int32, device="cuda") for _ in range(3)]
    hs = [torch.empty(shape.hidden, dtype=act_dtype(shape), device="cuda") for _ in range(3)]
    lgs = [torch.empty(shape.vocab, dtype=torch.float32, device="cuda") for _ in range(3)]
    cur_t, cur_h = tok, h_in
    for i in range(3):
        abi.mtp_draft_step(gh, gkv, cur_t, cur_h, hs[i], lgs[i], toks[i], ws)
        cur_t, cur_h = toks[i], hs[i]
    torch.cuda.synchronize()
    o_t, o_h = 5, I.decode(hid[0], shape.act_dtype)
    for i in range(3):
        ref = oh.step(okv, o_t, o_h)
        lg = host(lgs[i])
        assert rel_err(lg, ref["logits"]) <= tol, (i, rel_err(lg, ref["logits"]))
        assert rel_err(host(hs[i]), ref["g"][0]) <= tol, i
        assert argmax_ok(int(host(toks[i])[0]), ref["logits"], lg)[0], i
        assert int(host(toks[i])[0]) == int(np.argmax(lg))
        # teacher forcing: the next oracle step takes what the GPU fed its next step
        o_t, o_h = int(host(toks[i])[0]), np.asarray(host(hs[i]), np.float64)
    assert host(gkv.state)[0] == 203
    check_kv(gkv, okv, shape, 200, 203, tol)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("mode", [OH.KV_ONLY, OH.LAST, OH.ALL])
def test_flush_zero_pairs(name, mode):
    """A device count of 0 (nothing pending): no slot is written, the length
    stays, the round base is recorded at it, and the outputs are untouched --
    what the oracle's empty flush does."""
    from mtp_draft_head_step_amd import abi
    shape = SHAPES[name]
    wl, n_max, cap, prefix = 60, 3, 512, 200
    _, gh, oh = build(shape, wl)
    gkv, okv = kv_pair(shape, wl, prefix, cap)
    k0, v0 = host(gkv.k).copy(), host(gkv.v).copy()
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, n_max, cap))
    toks = I.tokens_uniform(wl, 1, n_max, shape.vocab)
    hids = I.target_hiddens(shape, wl, 1, n_max)
    hout = torch.zeros((n_max, shape.hidden), dtype=act_dtype(shape), device="cuda")
    logits = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    n_dev = torch.zeros(1, dtype=torch.int32, device="cuda")
    abi.mtp_flush_pairs(gh, gkv, device_array(toks), device_array(hids), n_max, n_dev, mode, 1,
                        hout if mode == OH.ALL else hout[:1], logits, amax, ws)
    torch.cuda.synchronize()
    assert oh.flush(okv, [], [], mode, set_round_base=True) == {}
    assert host(gkv.state).tolist() == [okv.len, okv.base, 0, 0] == [prefix, prefix, 0, 0]
    assert np.array_equal(host(gkv.k), k0) and np.array_equal(host(gkv.v), v0)
    assert np.all(host(logits) == 0) and int(host(amax)[0]) == -1 and np.all(host(hout) == 0)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("mode", [OH.KV_ONLY, OH.LAST, OH.ALL])
@pytest.mark.parametrize("n, n_max, use_dev", [(5, 5, False), (3, 8, True), (37, 40, True), (1, 1, False)])
def test_flush_parity(name, mode, n, n_max, use_dev):
    """Flush of n pairs (device count n <= host bound n_max when use_dev) in each
    output mode; more than 16 rows spans several row blocks of the GEMVs."""
    from mtp_draft_head_step_amd import abi
    shape = SHAPES[name]
    tol = tol_of(shape)
    wl = 70 + n
    _, gh, oh = build(shape, wl)
    cap = 1024
    prefix = 300
    gkv, okv = kv_pair(shape, wl, prefix, cap)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, n_max, cap))
    toks = I.tokens_uniform(wl, 1, n_max, shape.vocab)
    hids = I.target_hiddens(shape, wl, 1, n_max)
    hout = torch.zeros((n_max if mode == OH.ALL else 1, shape.hidden), dtype=act_dtype(shape), device="cuda")
    logits = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    n_dev = torch.tensor([n], dtype=torch.int32, device="cuda") if use_dev else None
    abi.mtp_flush_pairs(gh, gkv, device_array(toks), device_array(hids), n_max if use_dev else n,
                        n_dev, mode, 1, hout, logits, amax, ws)
    torch.cuda.synchronize()
    ref = oh.flush(okv, [int(t) for t in toks[:n]], [I.decode(h, shape.act_dtype) for h in hids[:n]],
                   mode, set_round_base=True)
    st = host(gkv.state)
    assert st[0] == prefix + n and st[1] == prefix + n and st[3] == 0
    check_kv(gkv, okv, shape, prefix, prefix + n, tol)
    if mode == OH.KV_ONLY:
        assert np.all(host(logits) == 0) and int(host(amax)[0]) == -1
        return
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol
    assert argmax_ok(int(host(amax)[0]), ref["logits"], lg)[0]
    g = host(hout)
    if mode == OH.ALL:
        for j in range(n):
            assert rel_err(g[j], ref["g"][j]) <= tol
        if n < n_max:
            assert np.all(g[n:] == 0)                 # rows beyond the device count untouched
    else:
        assert rel_err(g[0], ref["g"][0]) <= tol


@pytest.mark.parametrize("name", list(SHAPES))
def test_flush_equals_chain_on_gpu(name):
    """Block = chain (the pages' chain-parity contract) on the GPU: a 4-pair flush
    leaves the same K/V and last-row output as 4 steps, within the tolerance."""
    from mtp_draft_head_step_amd import abi
    shape = SHAPES[name]
    tol = tol_of(shape)
    _, gh, _ = build(shape, 80)
    cap = 256
    kv1, _ = kv_pair(shape, 80, 50, cap)
    kv2, _ = kv_pair(shape, 80, 50, cap)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, 4, cap))
    toks = device_array(I.tokens_uniform(80, 2, 4, shape.vocab))
    hids = device_array(I.target_hiddens(shape, 80, 2, 4))
    h1 = torch.empty((1, shape.hidden), dtype=act_dtype(shape), device="cuda")
    l1 = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    abi.mtp_flush_pairs(gh, kv1, toks, hids, 4, None, OH.LAST, 0, h1, l1, None, ws)
    h2 = torch.empty(shape.hidden, dtype=act_dtype(shape), device="cuda")
    l2 = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    for j in range(4):
        abi.mtp_draft_step(gh, kv2, toks[j:j + 1], hids[j], h2, l2, None, ws)
    torch.cuda.synchronize()
    assert rel_err(host(l1), host(l2)) <= tol
    assert_vectors(host(kv1.k)[:, 50:54], host(kv2.k)[:, 50:54], tol, "K")
    assert_vectors(host(kv1.v)[:, 50:54], host(kv2.v)[:, 50:54], tol, "V")


def test_capacity_and_count_errors_are_sticky():
    from mtp_draft_head_step_amd import abi
    shape = I.TINY_F32
    _, gh, _ = build(shape, 81)
    gkv, _ = kv_pair(shape, 81, 6, 8)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, 4, 8))
    toks = device_array(I.tokens_uniform(81, 3, 4, shape.vocab))
    hids = device_array(I.target_hiddens(shape, 81, 3, 4))
    hout = torch.empty((1, shape.hidden), dtype=torch.float32, device="cuda")
    n_bad = torch.tensor([5], dtype=torch.int32, device="cuda")          # above n_max = 4
    abi.mtp_flush_pairs(gh, gkv, toks, hids, 4, n_bad, OH.LAST, 0, hout, None, None, ws)
    torch.cuda.synchronize()
    assert host(gkv.state).tolist() == [6, 6, 0, abi.DEV_COUNT]
    gkv.state.copy_(torch.tensor([6, 6, 0, 0], dtype=torch.int32))
    abi.mtp_flush_pairs(gh, gkv, toks, hids, 4, None, OH.LAST, 0, hout, None, None, ws)   # 6 + 4 > 8
    torch.cuda.synchronize()
    assert host(gkv.state).tolist() == [6, 6, 0, abi.DEV_CAPACITY]
    abi.mtp_draft_step(gh, gkv, toks[:1], hids[0], hout[0], None, None, ws)           # no-op now
    abi.kv_rollback(gkv, 2)
    torch.cuda.synchronize()
    assert host(gkv.state).tolist() == [6, 6, 0, abi.DEV_CAPACITY]


@pytest.mark.parametrize("bad", [-1, 1024, 1 << 30])
def test_token_out_of_range_sets_error(bad):
    """A pair whose token is outside [0, vocab) is not read from the embedding
    table: the KV error word becomes MTP_DEV_TOKEN and nothing is appended."""
    from mtp_draft_head_step_amd import abi
    shape = I.TINY_F32
    _, gh, _ = build(shape, 82)
    gkv, _ = kv_pair(shape, 82, 6, 64)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, 4, 64))
    toks = I.tokens_uniform(82, 3, 4, shape.vocab)
    toks[2] = bad
    hids = device_array(I.target_hiddens(shape, 82, 3, 4))
    hout = torch.empty((1, shape.hidden), dtype=torch.float32, device="cuda")
    abi.mtp_flush_pairs(gh, gkv, device_array(toks), hids, 4, None, OH.LAST, 1, hout, None, None, ws)
    torch.cuda.synchronize()
    assert host(gkv.state).tolist() == [6, 6, 0, abi.DEV_TOKEN]


# head_dim 64, 128 and 256 with grouped heads 4 and 6, and a hidden size past
# the weight-streaming product's threshold: the matrix-core flush kernels at
# their other shapes (bf16 weights, activations and KV)
MID_SHAPES = {
    "d128_g4": I.HeadShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=1024,
                           vocab=2048).with_dtypes(weight_dtype=I.BF16, act_dtype=I.BF16, kv_dtype=I.BF16,
                                                   lm_head_dtype=I.BF16),
    "d256_g6": I.HeadShape(hidden=512, n_q_heads=6, n_kv_heads=1, head_dim=256, intermediate=1536,
                           vocab=2048).with_dtypes(weight_dtype=I.BF16, act_dtype=I.BF16, kv_dtype=I.BF16,
                                                   lm_head_dtype=I.BF16),
    "d64_g4": I.HeadShape(hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=64, intermediate=768,
                          vocab=2048).with_dtypes(weight_dtype=I.BF16, act_dtype=I.BF16, kv_dtype=I.BF16,
                                                  lm_head_dtype=I.BF16),
    # hidden 2048: fc, gate/up and down (4M+ weights) take the weight-streaming
    # product (split-K partials and the SwiGLU epilogue), q/k/v and o the tiles
    "h2048": I.HeadShape(hidden=2048, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=2048,
                         vocab=2048).with_dtypes(weight_dtype=I.BF16, act_dtype=I.BF16, kv_dtype=I.BF16,
                                                 lm_head_dtype=I.BF16),
    # 260 gate/up tiles over 256 workgroups: stream-K, nearly every tile cut
    # between two workgroups (head + tail pieces and the fixup)
    "i16640": I.HeadShape(hidden=512, n_q_heads=4, n_kv_heads=1, head_dim=128, intermediate=16640,
                          vocab=2048).with_dtypes(weight_dtype=I.BF16, act_dtype=I.BF16, kv_dtype=I.BF16,
                                                  lm_head_dtype=I.BF16),
}


@pytest.mark.parametrize("name", list(MID_SHAPES))
@pytest.mark.parametrize("n, n_max", [(17, 17), (70, 100), (130, 130)])
def test_flush_many_rows_parity(name, n, n_max):
    """ALL-mode flushes past 16 rows (the matrix-core projections and attention)
    at head_dim 128/256, every row's g, the last logits and the appended K/V."""
    from mtp_draft_head_step_amd import abi
    shape = MID_SHAPES[name]
    tol = tol_of(shape)
    wl = 90 + n
    _, gh, oh = build(shape, wl)
    cap, prefix = 1024, 333
    gkv, okv = kv_pair(shape, wl, prefix, cap)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, n_max, cap))
    toks = I.tokens_uniform(wl, 1, n_max, shape.vocab)
    hids = I.target_hiddens(shape, wl, 1, n_max)
    hout = torch.zeros((n_max, shape.hidden), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    n_dev = torch.tensor([n], dtype=torch.int32, device="cuda")
    abi.mtp_flush_pairs(gh, gkv, device_array(toks), device_array(hids), n_max, n_dev, OH.ALL, 1,
                        hout, logits, amax, ws)
    torch.cuda.synchronize()
    ref = oh.flush(okv, [int(t) for t in toks[:n]], [I.decode(h, shape.act_dtype) for h in hids[:n]],
                   OH.ALL, set_round_base=True)
    assert host(gkv.state).tolist() == [prefix + n, prefix + n, 0, 0]
    check_kv(gkv, okv, shape, prefix, prefix + n, tol)
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol
    assert argmax_ok(int(host(amax)[0]), ref["logits"], lg)[0]
    g = host(hout)
    for j in range(n):
        assert rel_err(g[j], ref["g"][j]) <= tol, j
    assert np.all(g[n:] == 0)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("n_draft", [1, 4])
def test_draft_chain_equals_flush_and_steps(name, n_draft):
    """mtp_draft_chain enqueues exactly the flush (LAST, round base) and the
    chained steps: drafts, hiddens, draft logits and the KV are bit-identical."""
    from mtp_draft_head_step_amd import abi
    shape = SHAPES[name]
    N = n_draft
    _, gh, _ = build(shape, 83)
    cap = 512
    kv1, _ = kv_pair(shape, 83, 200, cap)
    kv2, _ = kv_pair(shape, 83, 200, cap)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, 3, cap))
    toks = device_array(I.tokens_uniform(83, 4, 3, shape.vocab))
    hids = device_array(I.target_hiddens(shape, 83, 4, 3))
    n_dev = torch.tensor([2], dtype=torch.int32, device="cuda")
    dt = act_dtype(shape)
    d1 = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    g1 = torch.zeros((N, shape.hidden), dtype=dt, device="cuda")
    l1 = torch.zeros((N, shape.vocab), dtype=torch.float32, device="cuda")
    abi.mtp_draft_chain(gh, kv1, toks, hids, 3, n_dev, N, d1, g1, l1, ws)
    d2 = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    g2 = torch.zeros((N, shape.hidden), dtype=dt, device="cuda")
    l2 = torch.zeros((N, shape.vocab), dtype=torch.float32, device="cuda")
    abi.mtp_flush_pairs(gh, kv2, toks, hids, 3, n_dev, OH.LAST, 1, g2[0], l2[0], d2[0:1], ws)
    for i in range(1, N):
        abi.mtp_draft_step(gh, kv2, d2[i - 1:i], g2[i - 1], g2[i], l2[i], d2[i:i + 1], ws)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2) and torch.equal(g1, g2) and torch.equal(l1, l2)
    assert torch.equal(kv1.state, kv2.state) and int(host(kv1.state)[0]) == 200 + 2 + N - 1
    assert int(host(kv1.state)[1]) == 202
    assert torch.equal(kv1.k, kv2.k) and torch.equal(kv1.v, kv2.v)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_draft", [1, 2, 5])
def test_repair_pending(dtype, n_draft):
    """Device re-pairing under the keep-accepted policy: for every k the pending
    pairs are tokens[j0..k] and hidden rows j0..k with j0 = min(k, N-1)."""
    from mtp_draft_head_step_amd import abi
    N, H = n_draft, 96
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    code = abi.MTP_BF16 if dtype == "bf16" else abi.MTP_F32
    rng = np.random.default_rng(N)
    toks = torch.tensor(rng.integers(0, 1000, N + 1), dtype=torch.int32, device="cuda")
    hid = torch.tensor(rng.standard_normal((N + 1, H)), dtype=tdt, device="cuda")
    for k in range(N + 1):
        counts = torch.tensor([k, k + 1], dtype=torch.int32, device="cuda")
        pt = torch.full((N + 1,), -7, dtype=torch.int32, device="cuda")
        ph = torch.zeros((N + 1, H), dtype=tdt, device="cuda")
        pc = torch.zeros(1, dtype=torch.int32, device="cuda")
        abi.mtp_repair_pending(toks, counts, hid, H, code, N, pt, ph, pc)
        torch.cuda.synchronize()
        j0 = min(k, N - 1)
        c = k + 1 - j0
        assert int(pc.item()) == c and c == (1 if k < N else min(2, N + 1 - j0))
        assert torch.equal(pt[:c], toks[j0:k + 1]) and torch.all(pt[c:] == -7)
        assert torch.equal(ph[:c], hid[j0:k + 1])
