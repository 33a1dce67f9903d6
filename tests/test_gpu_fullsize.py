"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark times, through the C ABI:

* the Qwen3.5-27B-shaped head (H 5120, 24/4 heads, D 256, I 17408, V 152064,
  bf16) at a 4096-slot draft KV: one chained step and the in-round flush of up
  to three pending pairs (host bound 3, device count 2 or 3);
* the same head with an int8-g128 lm_head: a step and a 3-pair LAST flush;
* the 256-pair flush of the tiny head in bf16 over an 8192-slot prefix, in all
  three output modes;
* the tiny bf16 head over a 32768-slot prefix with a bf16 or an int8-g128
  lm_head: a step, and whole greedy rounds at depths 1, 2, 4 and 8 under both
  KV policies with the planted acceptance p_i = 0.8 * 0.85^i.

Every output is compared with the oracle element by element (logits, g, the
appended K/V); tokens, counts and KV lengths exactly.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mtp_draft_head_step_amd import inputs as I
from oracle import head as OH
from oracle import rounds as R
from oracle.kvcache import DraftKV
from tests.gpu_util import (argmax_ok, assert_vectors, compare_rounds, device_array, host, kv_pair,
                            rel_err, tol_of)

pytestmark = pytest.mark.gpu

QWEN_CTX = 4096
QWEN_CAP = QWEN_CTX + 256 + 32


@pytest.fixture(scope="module")
def qwen():
    """The 27B-shaped head on the GPU and in the oracle, with a 4096-slot prefix."""
    from mtp_draft_head_step_amd import abi
    shape, wl = I.QWEN35_27B, I.WL_QWEN
    st = I.head_weights(shape, wl)
    gh = abi.Head(shape, st)
    oh = OH.Head(shape, I.weight_values(shape, st), cache_fp64=True)
    del st
    kp, vp = I.prefix_kv(shape, wl, QWEN_CTX, QWEN_CAP)
    return {"shape": shape, "gh": gh, "oh": oh, "kp": kp, "vp": vp}


def _qwen_kv(q):
    from mtp_draft_head_step_amd import abi
    s = q["shape"]
    g = abi.DraftKV(s, QWEN_CAP, q["kp"], q["vp"], QWEN_CTX)
    o = DraftKV(s.n_kv_heads, QWEN_CAP, s.head_dim, I.decode(q["kp"], s.kv_dtype),
                I.decode(q["vp"], s.kv_dtype), QWEN_CTX)
    return g, o


def _check_slots(gkv, okv, lo, hi, tol):
    """Every K and V entry of slots [lo, hi), per head and slot."""
    assert_vectors(host(gkv.k)[:, lo:hi], okv.K[:, lo:hi], tol, "K")
    assert_vectors(host(gkv.v)[:, lo:hi], okv.V[:, lo:hi], tol, "V")


@pytest.mark.timeout(600)
def test_qwen27b_step_parity(qwen):
    """One draft step at slot 4096: logits over all 152064 rows, g, the fused
    argmax and the appended K/V."""
    from mtp_draft_head_step_amd import abi
    s, gh, oh = qwen["shape"], qwen["gh"], qwen["oh"]
    tol = tol_of(s)
    gkv, okv = _qwen_kv(qwen)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, 1, QWEN_CAP))
    tok = int(I.tokens_uniform(I.WL_QWEN, 900, 1, s.vocab)[0])
    hid = I.target_hiddens(s, I.WL_QWEN, 900, 1)
    hout = torch.empty(s.hidden, dtype=torch.bfloat16, device="cuda")
    logits = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    abi.mtp_draft_step(gh, gkv, torch.tensor([tok], dtype=torch.int32, device="cuda"),
                       device_array(hid[0]), hout, logits, amax, ws)
    torch.cuda.synchronize()
    ref = oh.step(okv, tok, I.decode(hid[0], s.act_dtype))
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol
    assert rel_err(host(hout), ref["g"][0]) <= tol
    assert argmax_ok(int(host(amax)[0]), ref["logits"], lg)[0]
    assert int(host(amax)[0]) == int(np.argmax(lg))
    assert host(gkv.state).tolist() == [QWEN_CTX + 1, QWEN_CTX, 0, 0]
    _check_slots(gkv, okv, QWEN_CTX - 2, QWEN_CTX + 1, tol)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n, n_max, mode", [(3, 3, OH.ALL), (2, 3, OH.LAST), (5, 5, OH.ALL), (8, 12, OH.ALL),
                                            (16, 16, OH.LAST)])
def test_qwen27b_flush_parity(qwen, n, n_max, mode):
    """The round's flush: host bound 3 rows (two drafts + one), device count n,
    round base recorded; ALL mode returns every row's g.  Past 4 rows the 27B
    head runs the MFMA products (5, 8 of 12, 16 rows)."""
    from mtp_draft_head_step_amd import abi
    s, gh, oh = qwen["shape"], qwen["gh"], qwen["oh"]
    tol = tol_of(s)
    gkv, okv = _qwen_kv(qwen)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, n_max, QWEN_CAP))
    toks = I.tokens_uniform(I.WL_QWEN, 901, n_max, s.vocab)
    hids = I.target_hiddens(s, I.WL_QWEN, 901, n_max)
    hout = torch.zeros((n_max if mode == OH.ALL else 1, s.hidden), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros(s.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    n_dev = torch.tensor([n], dtype=torch.int32, device="cuda")
    abi.mtp_flush_pairs(gh, gkv, device_array(toks), device_array(hids), n_max, n_dev, mode, 1,
                        hout, logits, amax, ws)
    torch.cuda.synchronize()
    ref = oh.flush(okv, [int(t) for t in toks[:n]], [I.decode(h, s.act_dtype) for h in hids[:n]],
                   mode, set_round_base=True)
    assert host(gkv.state).tolist() == [QWEN_CTX + n, QWEN_CTX + n, 0, 0]
    _check_slots(gkv, okv, QWEN_CTX, QWEN_CTX + n, tol)
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol
    assert argmax_ok(int(host(amax)[0]), ref["logits"], lg)[0]
    g = host(hout)
    rows = range(n) if mode == OH.ALL else [0]
    for j, r in enumerate(rows):
        assert rel_err(g[r], ref["g"][j]) <= tol
    if mode == OH.ALL:
        assert np.all(g[n:] == 0)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n_max, mode", [(3, OH.LAST), (8, OH.ALL)])
def test_qwen27b_flush_zero_pairs(qwen, n_max, mode):
    """The MFMA flush path with a device count of 0: nothing appended, the round
    base recorded at the unchanged length, the outputs untouched."""
    from mtp_draft_head_step_amd import abi
    s, gh = qwen["shape"], qwen["gh"]
    gkv, _ = _qwen_kv(qwen)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, n_max, QWEN_CAP))
    toks = I.tokens_uniform(I.WL_QWEN, 905, n_max, s.vocab)
    hids = I.target_hiddens(s, I.WL_QWEN, 905, n_max)
    hout = torch.zeros((n_max, s.hidden), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros(s.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    n_dev = torch.zeros(1, dtype=torch.int32, device="cuda")
    abi.mtp_flush_pairs(gh, gkv, device_array(toks), device_array(hids), n_max, n_dev, mode, 1,
                        hout if mode == OH.ALL else hout[:1], logits, amax, ws)
    torch.cuda.synchronize()
    assert host(gkv.state).tolist() == [QWEN_CTX, QWEN_CTX, 0, 0]
    assert not host(gkv.k)[:, QWEN_CTX:QWEN_CTX + n_max].any()
    assert np.all(host(logits) == 0) and int(host(amax)[0]) == -1 and np.all(host(hout) == 0)


@pytest.mark.timeout(900)
def test_qwen27b_flush256_parity(qwen):
    """The pages' full flush at the 27B shape: 256 pending pairs (2.5 MiB of bf16
    hiddens) after the 4096-slot prefix, ALL mode (the matrix-core path).  Every
    appended K/V slot, the last row's logits and argmax, and g at sampled rows
    (first, second, middle, last two) are compared with the oracle."""
    from mtp_draft_head_step_amd import abi
    s, gh, oh = qwen["shape"], qwen["gh"], qwen["oh"]
    tol = tol_of(s)
    gkv, okv = _qwen_kv(qwen)
    n = 256
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, n, QWEN_CAP))
    toks = I.tokens_uniform(I.WL_QWEN, 902, n, s.vocab)
    hids = I.target_hiddens(s, I.WL_QWEN, 902, n)
    hout = torch.zeros((n, s.hidden), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros(s.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    abi.mtp_flush_pairs(gh, gkv, device_array(toks), device_array(hids), n, None, OH.ALL, 1, hout, logits, amax,
                        ws)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 254, 255]
    ref = oh.flush(okv, [int(t) for t in toks], [I.decode(h, s.act_dtype) for h in hids], OH.ALL,
                   set_round_base=True, out_rows=rows)
    assert host(gkv.state).tolist() == [QWEN_CTX + n, QWEN_CTX + n, 0, 0]
    for lo in range(QWEN_CTX, QWEN_CTX + n, 64):
        _check_slots(gkv, okv, lo, lo + 64, tol)
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol
    assert argmax_ok(int(host(amax)[0]), ref["logits"], lg)[0]
    g = host(hout)
    for i, r in enumerate(rows):
        assert rel_err(g[r], ref["g"][i]) <= tol, r


@pytest.mark.timeout(1200)
def test_qwen27b_rounds_parity(qwen):
    """Whole greedy rounds at the 27B shape (two drafts, policy A), launched as
    the benchmark launches them.  Acceptance is planted so the rounds commit 1,
    2, 3 and 1 tokens: the rounds' flushes take 1, 1, 2 and 3 pending pairs with
    the device count from the previous verify, so the one-, two- and three-row
    flushes all run through mtp_draft_chain, spec_verify and kv_rollback.  Each
    round is compared with the oracle (draft logits and hiddens, drafts, k,
    tokens, KV lengths, every appended K/V entry)."""
    s, gh, oh = qwen["shape"], qwen["gh"], qwen["oh"]
    gkv, okv = _qwen_kv(qwen)
    N = 2
    plan = [0, 1, 2, 0]
    committed = I.tokens_uniform(I.WL_QWEN, 910, QWEN_CTX + 2, s.vocab)
    hid0 = I.target_hiddens(s, I.WL_QWEN, 911, 1)[0]

    def targets(rnd, drafts):
        rows = I.logits_rows(I.WL_QWEN, 5, (912, rnd), N + 1, s.vocab, 3.0)[0]
        I.plant_acceptance(rows, np.asarray(drafts, np.int64), plan[rnd])
        return rows, I.target_hiddens(s, I.WL_QWEN, (913, rnd), N + 1)

    ks, near = compare_rounds(gh, oh, gkv, okv, s, committed, hid0, N, targets, len(plan))
    assert ks == plan and near <= 1


@pytest.mark.timeout(900)
def test_batch_qwen27b_rounds(qwen):
    """Two sessions of the 27B-shaped head (prefixes 4096 and 4000) for three
    rounds with ragged planted acceptance: the flushes and steps of both
    sessions share one pass over the weights (matrix-core products for the
    flush and step projections, two-row unembedding)."""
    from tests.test_gpu_batch import batch_session, run_batch_rounds
    shape, gh, oh = qwen["shape"], qwen["gh"], qwen["oh"]
    cap = QWEN_CTX + 64
    gh, oh, gkv, states, hid0s = batch_session(shape, I.WL_QWEN, [QWEN_CTX, QWEN_CTX - 96], cap, gh=gh, oh=oh)
    plan = [[0, 2], [2, 1], [1, 0]]

    def targets(rnd, b, drafts_b):
        rows = I.logits_rows(I.WL_QWEN, 5, (930, rnd, b), 3, shape.vocab, 3.0)[0]
        I.plant_acceptance(rows, np.asarray(drafts_b, np.int64), plan[rnd][b])
        return rows, I.target_hiddens(shape, I.WL_QWEN, (931, rnd, b), 3)

    ks = run_batch_rounds(shape, gh, gkv, states, hid0s, 2, targets, 3, "A")
    assert ks == plan


@pytest.fixture(scope="module")
def qwen_i8():
    """The 27B-shaped head with its borrowed lm_head stored int8 per (row,
    128-column group) with fp16 scales (the quantised draft output head), on
    the GPU and in the oracle.  The other tensors are the bf16 head's."""
    from mtp_draft_head_step_amd import abi
    shape, wl = I.QWEN35_27B.with_dtypes(lm_head_dtype=I.I8G128), I.WL_QWEN
    st = I.head_weights(shape, wl)
    gh = abi.Head(shape, st)
    oh = OH.Head(shape, I.weight_values(shape, st), cache_fp64=True)
    del st
    kp, vp = I.prefix_kv(shape, wl, QWEN_CTX, QWEN_CAP)
    return {"shape": shape, "gh": gh, "oh": oh, "kp": kp, "vp": vp}


@pytest.mark.timeout(900)
def test_qwen27b_i8_lm_head_step_and_flush(qwen_i8):
    """The int8-g128 lm_head at the 27B shape (152064 x 5120 int8 + fp16 scales):
    one chained step (every logit, the fused argmax, g, the appended K/V) and
    the round's flush of 3 pairs in LAST mode (last row's logits and argmax)."""
    from mtp_draft_head_step_amd import abi
    s, gh, oh = qwen_i8["shape"], qwen_i8["gh"], qwen_i8["oh"]
    tol = tol_of(s)
    gkv, okv = _qwen_kv(qwen_i8)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, 3, QWEN_CAP))
    tok = int(I.tokens_uniform(I.WL_QWEN, 903, 1, s.vocab)[0])
    hid = I.target_hiddens(s, I.WL_QWEN, 903, 1)
    hout = torch.empty(s.hidden, dtype=torch.bfloat16, device="cuda")
    logits = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    abi.mtp_draft_step(gh, gkv, torch.tensor([tok], dtype=torch.int32, device="cuda"),
                       device_array(hid[0]), hout, logits, amax, ws)
    torch.cuda.synchronize()
    ref = oh.step(okv, tok, I.decode(hid[0], s.act_dtype))
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol
    assert rel_err(host(hout), ref["g"][0]) <= tol
    assert argmax_ok(int(host(amax)[0]), ref["logits"], lg)[0]
    assert int(host(amax)[0]) == int(np.argmax(lg))
    _check_slots(gkv, okv, QWEN_CTX, QWEN_CTX + 1, tol)

    toks = I.tokens_uniform(I.WL_QWEN, 904, 3, s.vocab)
    hids = I.target_hiddens(s, I.WL_QWEN, 904, 3)
    h1 = torch.zeros((1, s.hidden), dtype=torch.bfloat16, device="cuda")
    abi.mtp_flush_pairs(gh, gkv, device_array(toks), device_array(hids), 3, None, OH.LAST, 1,
                        h1, logits, amax, ws)
    torch.cuda.synchronize()
    ref = oh.flush(okv, [int(t) for t in toks], [I.decode(h, s.act_dtype) for h in hids], OH.LAST,
                   set_round_base=True)
    assert host(gkv.state).tolist() == [QWEN_CTX + 4, QWEN_CTX + 4, 0, 0]
    _check_slots(gkv, okv, QWEN_CTX + 1, QWEN_CTX + 4, tol)
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol
    assert rel_err(host(h1)[0], ref["g"][0]) <= tol
    assert argmax_ok(int(host(amax)[0]), ref["logits"], lg)[0]


# --------------------------------------------------------------------------
# 256-pair flush over an 8192-slot prefix (tiny head, bf16)
# --------------------------------------------------------------------------
@pytest.mark.timeout(300)
@pytest.mark.parametrize("mode", [OH.KV_ONLY, OH.LAST, OH.ALL])
def test_flush256_parity(mode):
    from mtp_draft_head_step_amd import abi
    shape, wl = I.TINY_BF16, I.WL_FLUSH
    tol = tol_of(shape)
    prefix, n, cap = 8192, 256, 8192 + 256
    st = I.head_weights(shape, wl)
    gh = abi.Head(shape, st)
    oh = OH.Head(shape, I.weight_values(shape, st))
    gkv, okv = kv_pair(shape, wl, prefix, cap)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, n, cap))
    toks = I.tokens_uniform(wl, 0, n, shape.vocab)
    hids = I.target_hiddens(shape, wl, 0, n)
    hout = torch.zeros((n if mode == OH.ALL else 1, shape.hidden), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    abi.mtp_flush_pairs(gh, gkv, device_array(toks), device_array(hids), n, None, mode, 1,
                        hout, logits, amax, ws)
    torch.cuda.synchronize()
    ref = oh.flush(okv, [int(t) for t in toks], [I.decode(h, shape.act_dtype) for h in hids],
                   mode, set_round_base=True)
    assert host(gkv.state).tolist() == [cap, cap, 0, 0]
    for lo in range(prefix, cap, 64):
        _check_slots(gkv, okv, lo, lo + 64, tol)
    if mode == OH.KV_ONLY:
        assert np.all(host(logits) == 0) and int(host(amax)[0]) == -1
        return
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol
    assert argmax_ok(int(host(amax)[0]), ref["logits"], lg)[0]
    g = host(hout)
    for j in range(g.shape[0]):
        assert rel_err(g[j], ref["g"][j]) <= tol, j


# --------------------------------------------------------------------------
# 32768-slot prefix, bf16 or int8-g128 lm_head, depth 1..8
# --------------------------------------------------------------------------
LONG_CTX = 32768
LONG_CAP = LONG_CTX + 64
LM_DTYPES = {"lm_bf16": I.BF16, "lm_i8g128": I.I8G128}


def _long_shape(lm):
    return I.TINY_BF16.with_dtypes(lm_head_dtype=LM_DTYPES[lm])


@pytest.mark.timeout(300)
@pytest.mark.parametrize("lm", list(LM_DTYPES))
def test_longctx_step_parity(lm):
    from mtp_draft_head_step_amd import abi
    shape, wl = _long_shape(lm), I.WL_DEPTH
    tol = tol_of(shape)
    st = I.head_weights(shape, wl)
    gh = abi.Head(shape, st)
    oh = OH.Head(shape, I.weight_values(shape, st))
    gkv, okv = kv_pair(shape, wl, LONG_CTX, LONG_CAP)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, 1, LONG_CAP))
    tok = int(I.tokens_uniform(wl, 0, 1, shape.vocab)[0])
    hid = I.target_hiddens(shape, wl, 0, 1)
    hout = torch.empty(shape.hidden, dtype=torch.bfloat16, device="cuda")
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    abi.mtp_draft_step(gh, gkv, torch.tensor([tok], dtype=torch.int32, device="cuda"),
                       device_array(hid[0]), hout, logits, amax, ws)
    torch.cuda.synchronize()
    ref = oh.step(okv, tok, I.decode(hid[0], shape.act_dtype))
    lg = host(logits)
    assert rel_err(lg, ref["logits"]) <= tol
    assert rel_err(host(hout), ref["g"][0]) <= tol
    assert argmax_ok(int(host(amax)[0]), ref["logits"], lg)[0]
    _check_slots(gkv, okv, LONG_CTX, LONG_CTX + 1, tol)


def _planted_target(shape, wl, rnd, n_draft):
    """Round ``rnd``'s target: N(0, 3) rows with greedy acceptance of the first
    k_r drafts planted (k_r drawn with p_i = 0.8 * 0.85^i), and N(0, 1) hiddens."""
    k_r = I.acceptance_draws(wl, rnd, n_draft)
    rows = I.logits_rows(wl, 5, rnd, n_draft + 1, shape.vocab, 3.0)[0]
    hid = I.target_hiddens(shape, wl, rnd, n_draft + 1)

    def fn(tokens, start):
        r = rows.copy()
        I.plant_acceptance(r, np.asarray(tokens[1:], np.int64), k_r)
        return r, I.decode(hid, shape.act_dtype)

    return k_r, hid, fn


@pytest.mark.timeout(300)
@pytest.mark.parametrize("lm", list(LM_DTYPES))
@pytest.mark.parametrize("policy", ["A", "B"])
@pytest.mark.parametrize("n_draft", [1, 2, 4, 8])
def test_depth_rounds_parity(lm, policy, n_draft):
    """Twelve greedy rounds over the 32768-slot prefix, launched as the benchmark
    launches them (mtp_draft_chain over the pending pairs with their device count,
    verify, rollback, device re-pairing under policy B); the planted acceptance
    fixes k, so k, the committed tokens, the re-paired pending pairs, the KV
    lengths and every appended K/V entry are compared with the oracle."""
    from mtp_draft_head_step_amd import abi
    shape, wl, N = _long_shape(lm), I.WL_DEPTH, n_draft
    tol = tol_of(shape)
    st = I.head_weights(shape, wl)
    gh = abi.Head(shape, st)
    oh = OH.Head(shape, I.weight_values(shape, st))
    gkv, okv = kv_pair(shape, wl, LONG_CTX, LONG_CAP)
    committed = [int(t) for t in I.tokens_uniform(wl, 1, LONG_CTX + 2, shape.vocab)]
    hid0 = I.target_hiddens(shape, wl, 1000, 1)
    ost = R.RoundState(oh, okv, [(committed[-1], I.decode(hid0[0], shape.act_dtype))], list(committed),
                       window=64)
    ws = abi.Workspace(abi.mtp_workspace_bytes(gh.cfg, N + 1, LONG_CAP))
    vws = abi.Workspace(abi.spec_verify_workspace_bytes(N, shape.vocab))
    ring = torch.zeros(64, dtype=torch.int32, device="cuda")
    ring_st = torch.zeros(2, dtype=torch.int32, device="cuda")
    d_buf = torch.zeros(N, dtype=torch.int32, device="cuda")
    g_buf = torch.zeros((N, shape.hidden), dtype=torch.bfloat16, device="cuda")
    out_t = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    out_c = torch.zeros(2, dtype=torch.int32, device="cuda")
    pend_t = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    pend_t[0] = committed[-1]
    pend_h = torch.zeros((N + 1, shape.hidden), dtype=torch.bfloat16, device="cuda")
    pend_h[0] = device_array(hid0[0])
    n_dev = torch.tensor([1], dtype=torch.int32, device="cuda")
    tgt_h = torch.zeros((N + 1, shape.hidden), dtype=torch.bfloat16, device="cuda")
    gpu_committed = list(committed)
    near_ties = 0
    for rnd in range(12):
        base = int(host(gkv.state)[0])
        # the round as the benchmark launches it: one drafting call, verify, rollback,
        # and (policy B) the device-side re-pairing
        abi.mtp_draft_chain(gh, gkv, pend_t, pend_h, N + 1, n_dev, N, d_buf, g_buf, None, ws)
        torch.cuda.synchronize()
        drafts = host(d_buf).tolist()
        k_r, hid_st, fn = _planted_target(shape, wl, rnd, N)
        rows, _ = fn([gpu_committed[-1]] + drafts, len(gpu_committed) - 1)
        tgt_h.copy_(device_array(hid_st))
        abi.spec_verify(abi.sampling(window=64), N, shape.vocab, device_array(rows), None, d_buf,
                        ring, ring_st, None, out_t, out_c, vws)
        torch.cuda.synchronize()
        appended = int(host(gkv.state)[0])
        abi.kv_rollback(gkv, abi.TO_ROUND_BASE, out_c[0:1] if policy == "B" else None, N)
        if policy == "B":
            abi.mtp_repair_pending(out_t, out_c, tgt_h, shape.hidden, abi.MTP_BF16, N, pend_t, pend_h, n_dev)
        else:
            pend_t[: N + 1] = out_t
            pend_h.copy_(tgt_h)
            n_dev.copy_(out_c[1:2])
        torch.cuda.synchronize()
        k = int(host(out_c)[0])
        assert k == k_r
        toks = host(out_t)[: k + 1].tolist()
        gpu_committed += toks
        j0 = 0 if policy == "A" else min(k, N - 1)
        assert int(host(n_dev)[0]) == k + 1 - j0
        assert host(pend_t)[: k + 1 - j0].tolist() == toks[j0:]
        # the oracle round follows the GPU's drafts; where they differ from the
        # oracle's argmax the oracle's top-two margin must be within the logits
        # tolerance (a near tie, where either token is correct)
        out = R.run_round(ost, N, fn, policy=policy, forced_drafts=drafts)
        for i, lg in enumerate(out["draft_logits"]):
            ref_tok = int(np.argmax(lg))
            if ref_tok != drafts[i]:
                near_ties += 1
                assert lg[ref_tok] - lg[drafts[i]] <= 2 * tol * np.max(np.abs(lg)), (rnd, i)
        assert out["k"] == k_r and out["tokens"] == toks
        st_now = host(gkv.state)
        assert st_now[3] == 0
        assert st_now[0] == ost.kv.len and st_now[1] == ost.kv.base
        # every entry the round appended (flushed pairs and chained drafts)
        _check_slots(gkv, ost.kv, base, appended, tol)
    assert gpu_committed == ost.committed
    assert near_ties <= 2
