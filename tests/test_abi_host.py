"""The C ABI on the host: libmtp.so loads, exports every function include/mtp.h
declares, and rejects bad arguments before anything is enqueued (these calls
return before any HIP call, so they run without a GPU)."""
import ctypes as C
import os
import re

import pytest

from mtp_draft_head_step_amd import abi
from mtp_draft_head_step_amd import inputs as I

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mtp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(abi.EXPORTS), names
    lib = C.CDLL(abi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert abi.mtp_status_string(0) == "MTP_OK"
    assert abi.mtp_status_string(-3) == "MTP_E_NOT_BOUND"
    assert abi.mtp_status_string(-99) == "MTP_E_UNKNOWN"


def fake_weights(shape, missing=()):
    w = abi.mtp_head_weights()
    for i, n in enumerate(abi.WEIGHT_FIELDS):
        if n not in missing:
            setattr(w, n, 0x10000 + 0x100 * i)      # never dereferenced on the host
    return w


def create(shape, w):
    h = C.c_void_p()
    st = abi.lib.mtp_head_create(C.byref(abi.config_of(shape)), C.byref(w), C.byref(h))
    if st == 0:
        abi.lib.mtp_head_destroy(h)
    return st


def test_create_validates():
    s = I.TINY_F32
    assert create(s, fake_weights(s, missing=("lm_head_scales",))) == abi.MTP_OK
    assert create(s, fake_weights(s, missing=("embed",))) == abi.MTP_E_NOT_BOUND      # not bound
    assert create(s, fake_weights(s, missing=("lm_head",))) == abi.MTP_E_NOT_BOUND
    assert create(s, fake_weights(s, missing=("k_norm",))) == abi.MTP_E_INVALID_ARG
    assert create(s.with_dtypes(head_dim=96), fake_weights(s)) == abi.MTP_E_UNSUPPORTED
    assert create(s.with_dtypes(n_q_heads=5), fake_weights(s)) == abi.MTP_E_UNSUPPORTED
    assert create(s.with_dtypes(n_q_heads=20, n_kv_heads=2), fake_weights(s)) == abi.MTP_E_UNSUPPORTED
    assert create(s.with_dtypes(hidden=200), fake_weights(s)) == abi.MTP_E_UNSUPPORTED
    assert create(s.with_dtypes(rms_eps=-1.0), fake_weights(s)) == abi.MTP_E_INVALID_ARG
    q = s.with_dtypes(lm_head_dtype="i8g128")
    assert create(q, fake_weights(q, missing=("lm_head_scales",))) == abi.MTP_E_INVALID_ARG
    assert create(q, fake_weights(q)) == abi.MTP_OK
    assert create(I.QWEN35_27B, fake_weights(I.QWEN35_27B)) == abi.MTP_OK


def test_workspace_sizes():
    cfg = abi.config_of(I.QWEN35_27B)
    a = abi.mtp_workspace_bytes(cfg, 1, 4608)
    b = abi.mtp_workspace_bytes(cfg, 3, 4608)
    assert 0 < a < b
    assert abi.mtp_workspace_bytes(cfg, 0, 4608) == 0
    assert abi.mtp_workspace_bytes(cfg, 257, 4608) == 0
    assert abi.spec_verify_workspace_bytes(4, 152064) > 0
    assert abi.spec_verify_workspace_bytes(17, 152064) == 0


def test_rollback_and_flush_fail_closed():
    kv = abi.mtp_kv(0x1000, 0x2000, 128, 0x3000)
    st = abi.lib.kv_rollback(C.byref(kv), 129, None, 2, None)
    assert st == abi.MTP_E_CAPACITY
    assert abi.lib.kv_rollback(C.byref(kv), -2, None, 2, None) == abi.MTP_E_INVALID_ARG
    assert abi.lib.kv_rollback(C.byref(kv), 5, 0x4000, 2, None) == abi.MTP_E_INVALID_ARG
    assert abi.lib.kv_rollback(C.byref(kv), -1, None, 17, None) == abi.MTP_E_INVALID_ARG
    bad = abi.mtp_kv(0, 0x2000, 128, 0x3000)

    s = I.TINY_F32
    h = C.c_void_p()
    assert abi.lib.mtp_head_create(C.byref(abi.config_of(s)), C.byref(fake_weights(s)), C.byref(h)) == 0
    try:
        ws = 1 << 40
        f = abi.lib.mtp_flush_pairs
        assert f(h, C.byref(kv), 0x10, 0x20, 257, None, 1, 0, 0x30, None, None, 0x40, ws, None) == abi.MTP_E_CAPACITY
        assert f(h, C.byref(kv), 0x10, 0x20, 0, None, 1, 0, 0x30, None, None, 0x40, ws, None) == abi.MTP_E_INVALID_ARG
        assert f(h, C.byref(kv), 0x10, 0x20, 4, None, 7, 0, 0x30, None, None, 0x40, ws, None) == abi.MTP_E_INVALID_ARG
        assert f(h, C.byref(kv), 0x10, 0x20, 4, None, 1, 0, 0x30, None, None, 0x40, 16, None) == abi.MTP_E_WORKSPACE
        assert f(h, C.byref(bad), 0x10, 0x20, 4, None, 1, 0, 0x30, None, None, 0x40, ws, None) == abi.MTP_E_INVALID_ARG
        small = abi.mtp_kv(0x1000, 0x2000, 3, 0x3000)
        assert f(h, C.byref(small), 0x10, 0x20, 4, None, 1, 0, 0x30, None, None, 0x40, ws, None) == abi.MTP_E_CAPACITY
        d = abi.lib.mtp_draft_step
        assert d(h, C.byref(kv), None, 0x20, 0x30, None, None, 0x40, ws, None) == abi.MTP_E_INVALID_ARG
        assert d(h, C.byref(kv), 0x10, 0x20, 0x20, None, None, 0x40, ws, None) == abi.MTP_E_INVALID_ARG
        assert d(h, C.byref(kv), 0x10, 0x20, 0x30, None, None, 0x40, 8, None) == abi.MTP_E_WORKSPACE
    finally:
        abi.lib.mtp_head_destroy(h)


def test_verify_fails_closed():
    v = abi.lib.spec_verify
    ws = 1 << 30
    greedy = abi.sampling()
    sampled = abi.sampling(0.7, 1.1, 40, 0.9, 0.05, 64)
    args = dict(t=0x10, d=0x20, dt=0x30, h=0x40, hs=0x50, u=0x60, ot=0x70, oc=0x80, ws=0x90)
    def call(sp, n, vocab, draft=0x20, u=0x60, wsb=ws):
        return v(C.byref(sp), n, vocab, 0x10, draft, 0x30, 0x40, 0x50, u, 0x70, 0x80, 0x90, wsb, None)
    assert call(greedy, 17, 100, draft=None) == abi.MTP_E_INVALID_ARG
    assert call(greedy, 2, 100, draft=0x20) == abi.MTP_E_INVALID_ARG     # greedy takes no draft rows
    assert call(sampled, 2, 100, draft=None) == abi.MTP_E_INVALID_ARG    # sampled needs them
    assert call(sampled, 2, 100, u=None) == abi.MTP_E_INVALID_ARG
    assert call(greedy, 2, 100, draft=None, wsb=8) == abi.MTP_E_WORKSPACE
    negative_k = abi.sampling(0.7, 1.0, -1, 0.9, 0.0, 64)
    assert call(negative_k, 2, 100) == abi.MTP_E_INVALID_ARG
    bad_win = abi.sampling(window=0)
    assert call(bad_win, 2, 100, draft=None) == abi.MTP_E_INVALID_ARG


def test_verify_rollback_fails_closed():
    """The fused verify + rollback checks the rollback's arguments as kv_rollback
    does and the verification's as spec_verify does, before any launch."""
    v = abi.lib.spec_verify_rollback
    greedy = abi.sampling()
    kv = abi.mtp_kv(0x1000, 0x2000, 128, 0x3000)
    no_state = abi.mtp_kv(0x1000, 0x2000, 128, 0)
    def call(kvd, to_len, keep, n=2, wsb=1 << 30, draft=None):
        return v(C.byref(greedy), n, 100, 0x10, draft, 0x30, 0x40, 0x50, None, 0x70, 0x80, 0x90, wsb,
                 C.byref(kvd) if kvd is not None else None, to_len, keep, 0xa0, None)
    assert call(kv, 129, 0) == abi.MTP_E_CAPACITY
    assert call(kv, -2, 0) == abi.MTP_E_INVALID_ARG
    assert call(kv, 5, 1) == abi.MTP_E_INVALID_ARG           # keep_accepted only with the round base
    assert call(kv, abi.TO_ROUND_BASE, 2) == abi.MTP_E_INVALID_ARG
    assert call(no_state, abi.TO_ROUND_BASE, 0) == abi.MTP_E_INVALID_ARG
    assert call(None, abi.TO_ROUND_BASE, 0) == abi.MTP_E_INVALID_ARG
    assert call(kv, abi.TO_ROUND_BASE, 0, n=17) == abi.MTP_E_INVALID_ARG
    assert call(kv, abi.TO_ROUND_BASE, 0, wsb=8) == abi.MTP_E_WORKSPACE
    assert call(kv, abi.TO_ROUND_BASE, 0, draft=0x20) == abi.MTP_E_INVALID_ARG


def test_static_step_rejects_oversized_scratch_on_host():
    """The no-workspace draft step refuses, before any HIP call, a step whose
    scratch would not fit the library's static array (4 MiB per device)."""
    big = I.HeadShape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=1 << 20, vocab=1024)
    assert abi.lib.mtp_workspace_bytes(C.byref(abi.config_of(big)), 1, 256) > (4 << 20)
    h = C.c_void_p()
    assert abi.lib.mtp_head_create(C.byref(abi.config_of(big)), C.byref(fake_weights(big)), C.byref(h)) == 0
    try:
        kv = abi.mtp_kv(0x1000, 0x2000, 256, 0x3000)
        st = abi.lib.mtp_draft_step_static(h, C.byref(kv), 0x4000, 0x5000, 0x6000, None, None, None)
        assert st == abi.MTP_E_WORKSPACE
        assert abi.lib.mtp_draft_step_static(None, C.byref(kv), 0x4000, 0x5000, 0x6000, None, None,
                                             None) == abi.MTP_E_INVALID_ARG
    finally:
        abi.lib.mtp_head_destroy(h)


def test_batch_calls_fail_closed_on_the_host():
    """The batched calls reject a batch outside 1..MTP_MAX_BATCH, a bad count
    stride and a short workspace before anything is enqueued."""
    s = I.TINY_F32
    cfg = abi.config_of(s)
    assert abi.lib.mtp_batch_workspace_bytes(C.byref(cfg), 0, 3, 256) == 0
    assert abi.lib.mtp_batch_workspace_bytes(C.byref(cfg), 17, 3, 256) == 0
    one = abi.lib.mtp_batch_workspace_bytes(C.byref(cfg), 1, 3, 256)
    four = abi.lib.mtp_batch_workspace_bytes(C.byref(cfg), 4, 3, 256)
    assert 0 < one < four
    h = C.c_void_p()
    assert abi.lib.mtp_head_create(C.byref(cfg), C.byref(fake_weights(s)), C.byref(h)) == 0
    try:
        kv = abi.mtp_kv(0x1000, 0x2000, 256, 0x3000)
        args = lambda b, stride, ws: (h, C.byref(kv), b, 0x4000, 0x5000, 3, 0x6000, stride, 2, 0x7000, 0x8000000,
                                      None, 0x9000, ws, None)
        f = abi.lib.mtp_draft_chain_batch
        assert f(*args(17, 1, four)) == abi.MTP_E_INVALID_ARG
        assert f(*args(0, 1, four)) == abi.MTP_E_INVALID_ARG
        assert f(*args(4, 0, four)) == abi.MTP_E_INVALID_ARG
        assert f(*args(4, 1, four - 1)) == abi.MTP_E_WORKSPACE
        sp = abi.sampling()
        v = abi.lib.spec_verify_batch
        per = abi.lib.spec_verify_workspace_bytes(2, 1000)
        assert v(C.byref(sp), 17, 2, 1000, 0x1, None, 0x2, 0x3, 0x4, None, 0x5, 0x6, 0x7, 17 * per, None) == \
            abi.MTP_E_INVALID_ARG
        assert v(C.byref(sp), 3, 2, 1000, 0x1, None, 0x2, 0x3, 0x4, None, 0x5, 0x6, 0x7, 3 * per - 1, None) == \
            abi.MTP_E_WORKSPACE
        assert abi.lib.kv_rollback_batch(C.byref(kv), 17, -1, None, 2, None) == abi.MTP_E_INVALID_ARG
        assert abi.lib.kv_rollback_batch(C.byref(kv), 2, 5, 0x10, 2, None) == abi.MTP_E_INVALID_ARG
        assert abi.lib.mtp_repair_pending_batch(17, 0x1, 0x2, 0x3, 256, abi.MTP_F32, 2, 0x4, 0x900000, 0x5,
                                                None) == abi.MTP_E_INVALID_ARG
    finally:
        abi.lib.mtp_head_destroy(h)
