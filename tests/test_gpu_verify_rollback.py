"""GPU parity of spec_verify_rollback (verification with the draft-KV rollback
and the round's report row in its final kernel) through the C ABI: the same
outputs as spec_verify followed by kv_rollback on the same inputs, the KV
state words the oracle's rollback gives for the verified k, and the report
row, in device memory and in host-coherent pinned memory."""
import ctypes as C

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import verify as OV
from oracle.kvcache import DraftKV
from mtp_draft_head_step_amd import inputs as I
from tests.gpu_util import device_array, host

pytestmark = pytest.mark.gpu

SENTINEL = -7


def make_case(rng, mode, vocab, n):
    rows = (rng.standard_normal((n + 1, vocab)) * 3).astype(np.float32)
    drafts = rng.integers(0, vocab, n).astype(np.int32)
    if mode == "greedy":
        I.plant_acceptance(rows, drafts.astype(np.int64), int(rng.integers(0, n + 1)), spike=20.0)
        return rows, None, drafts, None
    drows = (rows[:n] + 0.7 * rng.standard_normal((n, vocab))).astype(np.float32)
    # drafts with high draft probability, so both accepts and rejects occur
    for i in range(n):
        drafts[i] = int(np.argsort(drows[i])[-1 - int(rng.integers(0, 3))])
    u = rng.random(n + 1).astype(np.float32)
    return rows, drows, drafts, u


def sampling(mode):
    from mtp_draft_head_step_amd import abi
    if mode == "greedy":
        return abi.sampling(repeat_penalty=1.1, window=16), OV.Sampling(repeat_penalty=1.1, window=16)
    top_k = 40 if mode == "sampled" else 0
    return (abi.sampling(0.8, 1.1, top_k, 0.9, 0.05, 16),
            OV.Sampling(temperature=0.8, repeat_penalty=1.1, top_k=top_k, top_p=0.9, min_p=0.05, window=16))


def run(mode, rows, drows, drafts, u, ring, rst, kv_state, fused, to_len, keep, report=None):
    """One verification plus rollback; -> device outputs as host arrays."""
    from mtp_draft_head_step_amd import abi
    n, vocab = len(drafts), rows.shape[1]
    sp, _ = sampling(mode)
    ws = abi.Workspace(abi.spec_verify_workspace_bytes(n, vocab))
    t_ring, t_rst = device_array(ring), device_array(rst)
    out_t = torch.full((n + 1,), SENTINEL, dtype=torch.int32, device="cuda")
    out_c = torch.full((2,), SENTINEL, dtype=torch.int32, device="cuda")
    kv = abi.DraftKV(I.TINY_F32, 64)
    kv.state.copy_(torch.tensor(kv_state, dtype=torch.int32))
    state = kv.state
    args = (sp, n, vocab, device_array(rows), None if drows is None else device_array(drows),
            device_array(drafts) if n else None, t_ring, t_rst, None if u is None else device_array(u), out_t, out_c,
            ws)
    if fused:
        abi.spec_verify_rollback(*args, kv, to_len, keep, report)
    else:
        abi.spec_verify(*args)
        abi.kv_rollback(kv, to_len, out_c[0:1] if keep else None, n)
    torch.cuda.synchronize()
    return {"tokens": host(out_t), "counts": host(out_c), "ring": host(t_ring), "rst": host(t_rst),
            "state": host(state)}


# (KV state words before, to_len, keep_accepted)
ROLLBACKS = [
    ([40, 37, 0, 0], -1, 0),      # policy A: back to the round base
    ([40, 37, 0, 0], -1, 1),      # policy B: keep the accepted chained entries
    ([40, 37, 0, 0], 12, 0),      # an explicit length
    ([40, 37, 0, 0], 41, 0),      # past the length: error word 2, length kept
    ([40, 37, 0, 1], -1, 0),      # error word already set: nothing moves
]


@pytest.mark.parametrize("mode,vocab,n", [("greedy", 152064, 2), ("greedy", 1000, 4), ("greedy", 97, 0),
                                          ("sampled", 20000, 3), ("full", 4097, 2)])
@pytest.mark.parametrize("rb", range(len(ROLLBACKS)))
def test_fused_equals_verify_then_rollback(mode, vocab, n, rb):
    from mtp_draft_head_step_amd import abi
    st0, to_len, keep = ROLLBACKS[rb]
    rng = np.random.default_rng([vocab, n, rb, len(mode)])
    for trial in range(2):
        rows, drows, drafts, u = make_case(rng, mode, vocab, n)
        ring = rng.integers(0, vocab, 16).astype(np.int32)
        rst = np.array([int(rng.integers(0, 16)), int(rng.integers(0, 17))], np.int32)
        report = torch.full((6 + n + 1,), SENTINEL, dtype=torch.int32, device="cuda")
        a = run(mode, rows, drows, drafts, u, ring, rst, st0, True, to_len, keep, report)
        b = run(mode, rows, drows, drafts, u, ring, rst, st0, False, to_len, keep)
        k = int(a["counts"][0])
        assert 0 <= k <= n and a["counts"].tolist() == [k, k + 1] == b["counts"].tolist()
        assert np.array_equal(a["tokens"], b["tokens"])                 # untouched entries too
        assert np.array_equal(a["ring"], b["ring"]) and np.array_equal(a["rst"], b["rst"])
        assert a["state"].tolist() == b["state"].tolist()
        # the rollback the oracle makes for the verified k
        o = DraftKV(1, 64, 1, length=st0[0])
        o.base, o.err = st0[1], st0[3]
        o.rollback(to_len, k if keep else None, n)
        assert a["state"].tolist() == [o.len, o.base, st0[2], o.err]
        rep = host(report)
        assert rep[:6].tolist() == a["state"].tolist() + [k, k + 1]
        assert rep[6:6 + k + 1].tolist() == a["tokens"][:k + 1].tolist()
        assert (rep[6 + k + 1:] == SENTINEL).all()
        if mode == "greedy":                                            # and the verification itself
            _, sp_o = sampling(mode)
            ref = OV.verify(sp_o, rows, None, list(drafts), ring, rst)
            assert k == ref["k"] and a["tokens"][:k + 1].tolist() == ref["tokens"]


class CoherentRows:
    """Host-coherent pinned int32 rows (hipHostMalloc with the coherent flag,
    through the HIP runtime libmtp is bound to)."""

    def __init__(self, rows, cols):
        from mtp_draft_head_step_amd import abi
        self.hip = C.CDLL(abi.LIB_PATH)
        self.hip.hipHostMalloc.argtypes = [C.POINTER(C.c_void_p), C.c_size_t, C.c_uint]
        self.hip.hipHostFree.argtypes = [C.c_void_p]
        self.ptr = C.c_void_p()
        assert self.hip.hipHostMalloc(C.byref(self.ptr), rows * cols * 4, 0x40000000) == 0
        self.cols = cols
        self.view = np.ctypeslib.as_array((C.c_int32 * (rows * cols)).from_address(self.ptr.value)).reshape(rows,
                                                                                                            cols)
        self.view[:] = SENTINEL

    def addr(self, r):
        return self.ptr.value + r * self.cols * 4

    def close(self):
        self.hip.hipHostFree(self.ptr)


def test_report_rows_in_host_coherent_memory():
    """Rounds enqueued back to back, each writing its report row into host-
    coherent memory: after one synchronisation every row equals the device's
    outputs of its round (verify outputs compared on device copies)."""
    from mtp_draft_head_step_amd import abi
    n, vocab, rounds = 2, 152064, 6
    rng = np.random.default_rng(5)
    sp, _ = sampling("greedy")
    ws = abi.Workspace(abi.spec_verify_workspace_bytes(n, vocab))
    ring = device_array(np.zeros(16, np.int32))
    rst = device_array(np.zeros(2, np.int32))
    kv = abi.DraftKV(I.TINY_F32, 256)
    kv.state.copy_(torch.tensor([100, 90, 0, 0], dtype=torch.int32))
    state = kv.state
    rows = []
    for r in range(rounds):
        t, _, d, _ = make_case(rng, "greedy", vocab, n)
        rows.append((device_array(t), device_array(d)))
    out_t = torch.zeros((rounds, n + 1), dtype=torch.int32, device="cuda")
    out_c = torch.zeros((rounds, 2), dtype=torch.int32, device="cuda")
    snap = torch.zeros((rounds, 4), dtype=torch.int32, device="cuda")
    hrows = CoherentRows(rounds, 6 + n + 1)
    try:
        for r in range(rounds):
            t, d = rows[r]
            abi.spec_verify_rollback(sp, n, vocab, t, None, d, ring, rst, None, out_t[r], out_c[r], ws, kv,
                                     abi.TO_ROUND_BASE, r % 2 == 1, hrows.addr(r))
            snap[r].copy_(state)
            state[0] += 3                                   # the next round's appends
        torch.cuda.synchronize()
        ot, oc, sn = host(out_t), host(out_c), host(snap)
        for r in range(rounds):
            k = int(oc[r, 0])
            row = hrows.view[r]
            assert row[:6].tolist() == sn[r].tolist() + [k, k + 1]
            assert row[6:6 + k + 1].tolist() == ot[r, :k + 1].tolist()
            assert (row[6 + k + 1:] == SENTINEL).all()
    finally:
        hrows.close()
