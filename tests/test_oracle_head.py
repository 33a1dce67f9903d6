"""Pins for the oracle's head forward: closed forms, special cases that reduce to
hand-computable values, and invariants.  CPU only."""
import math

import numpy as np
import pytest

from mtp_draft_head_step_amd import inputs as I
from oracle import head as H
from oracle.kvcache import DraftKV


# ---------------------------------------------------------------- primitives
def test_rmsnorm_closed_form():
    y = H.rmsnorm([3.0, 4.0], [1.0, 1.0], 0.0)
    # mean square 12.5 -> divide by sqrt(12.5)
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    y = H.rmsnorm([3.0, 4.0], [2.0, -1.0], 0.0)
    assert np.allclose(y, [6 / math.sqrt(12.5), -4 / math.sqrt(12.5)], atol=1e-15)
    # eps enters inside the root: x = [1, 1], eps = 3 -> 1 / 2
    assert np.allclose(H.rmsnorm([1.0, 1.0], [1.0, 1.0], 3.0), [0.5, 0.5], atol=1e-15)
    # zero vector stays zero
    assert np.all(H.rmsnorm(np.zeros(8), np.ones(8), 1e-6) == 0)


def test_rmsnorm_scale_invariance():
    x = np.random.default_rng(0).standard_normal(64)
    a = H.rmsnorm(x, np.ones(64), 0.0)
    b = H.rmsnorm(7.5 * x, np.ones(64), 0.0)
    assert np.allclose(a, b, atol=1e-14)
    assert abs(np.mean(a * a) - 1.0) < 1e-13


def test_rope_closed_forms():
    # D = 2: one pair, inverse frequency 1, rotation by pos radians
    assert np.allclose(H.rope([1.0, 0.0], 3, 1e6), [math.cos(3), math.sin(3)], atol=1e-15)
    # D = 4, theta = 100: pairs (0, 2) at pos * 1 and (1, 3) at pos * 100^(-1/2) = pos * 0.1
    assert np.allclose(H.rope([0.0, 1.0, 0.0, 0.0], 5, 100.0),
                       [0.0, math.cos(0.5), 0.0, math.sin(0.5)], atol=1e-15)
    assert np.allclose(H.rope([1.0, 0.0, 0.0, 0.0], 5, 100.0),
                       [math.cos(5), 0.0, math.sin(5), 0.0], atol=1e-15)
    x = np.random.default_rng(1).standard_normal(64)
    assert np.array_equal(H.rope(x, 0, 1e6), x)                       # position 0: identity


def test_rope_relative_position():
    r = np.random.default_rng(2)
    q, k = r.standard_normal(64), r.standard_normal(64)
    a = H.rope(q, 17, 1e4) @ H.rope(k, 10, 1e4)
    b = H.rope(q, 107, 1e4) @ H.rope(k, 100, 1e4)
    assert abs(a - b) < 1e-11
    # pair norms are preserved
    y = H.rope(q, 1234, 1e6)
    assert np.allclose(q[:32] ** 2 + q[32:] ** 2, y[:32] ** 2 + y[32:] ** 2, atol=1e-12)


def test_silu_values():
    assert H.silu(0.0) == 0.0
    assert abs(H.silu(1.0) - 0.7310585786300049) < 1e-15               # 1 / (1 + e^-1)
    assert abs(H.silu(40.0) - 40.0) < 1e-12
    assert abs(H.silu(-40.0)) < 1e-15


def test_matvec_special_cases():
    x = np.arange(6, dtype=np.float64)
    assert np.array_equal(H.matvec(np.eye(6, dtype=np.float32), x), x)
    assert np.array_equal(H.matvec(np.ones((3, 6), np.float32), x), [15.0, 15.0, 15.0])
    w = np.zeros((20000, 6), np.float32)
    w[19999, 5] = 2.0
    y = H.matvec(w, x)                                                   # crosses a row block
    assert y[19999] == 10.0 and np.count_nonzero(y) == 1


def test_attend_two_keys_logistic():
    # scores a*b/sqrt(D) and 0 -> weights sigmoid(ab/sqrt(D)), 1 - sigmoid
    d = 4
    q = np.zeros((1, d)); q[0, 0] = 2.0
    K = np.zeros((1, 3, d)); K[0, 0, 0] = 1.5
    V = np.zeros((1, 3, d)); V[0, 0] = [1, 2, 3, 4]; V[0, 1] = [-1, 0, 5, 0]
    o = H.attend(q, K, V, 2)
    sig = 1.0 / (1.0 + math.exp(-3.0 / 2.0))
    assert np.allclose(o[0], sig * V[0, 0] + (1 - sig) * V[0, 1], atol=1e-14)


def test_attend_gqa_grouping_and_uniform():
    # q = 0 -> uniform weights -> mean of V over the visible keys; q-heads 0,1 read kv 0, 2,3 read kv 1
    r = np.random.default_rng(3)
    K = r.standard_normal((2, 8, 4)); V = r.standard_normal((2, 8, 4))
    o = H.attend(np.zeros((4, 4)), K, V, 5)
    for h in range(4):
        assert np.allclose(o[h], V[h // 2, :5].mean(axis=0), atol=1e-14)


def test_dequant_bound():
    w = np.random.default_rng(4).standard_normal((8, 256)).astype(np.float32) * 0.02
    w[3, 128:] = 0.0
    q, s = I.quantize_i8g128(w)
    d = H.dequant_i8g128(q, s)
    s64 = np.repeat(s.astype(np.float64), 128, axis=1)
    # |w - q s| <= s / 2 (+ the fp16 rounding of s times |q| <= 127)
    err = np.abs(w - d)
    bound = s64 / 2 + 127 * np.abs(s64 - (np.abs(w).reshape(8, 2, 128).max(2).repeat(128, 1) / 127))
    assert np.all(err <= bound + 1e-12)
    assert np.all(q[3, 128:] == 0) and s[3, 1] == 0
    assert np.abs(q).max() <= 127


# ---------------------------------------------------------------- structured heads
SMALL = I.HeadShape(hidden=8, n_q_heads=2, n_kv_heads=1, head_dim=4, intermediate=8, vocab=16)


def zero_head(shape=SMALL):
    sh = I.tensor_shapes(shape)
    w = {n: np.zeros(s, np.float32) for n, s in sh.items()}
    for n in I.NORM_TENSORS:
        w[n] = np.ones(sh[n], np.float32)
    r = np.random.default_rng(5)
    w["embed"] = r.standard_normal(sh["embed"]).astype(np.float32)
    w["lm_head"] = np.zeros(sh["lm_head"], np.float32)
    w["lm_head"][: shape.hidden] = np.eye(shape.hidden, dtype=np.float32)
    return w


def test_zero_fc_gives_mean_of_values():
    """fc = 0: x = 0, so q = k = v = 0 at the new slot; the new query attends
    uniformly; with o_proj = I and a zero MLP, g = mean(V[0..S]) (the new zero
    value included) and logits[:H] = RMSNorm(g)."""
    w = zero_head()
    w["o_proj"] = np.eye(8, dtype=np.float32)
    hd = H.Head(SMALL, w)
    r = np.random.default_rng(6)
    Kp, Vp = r.standard_normal((1, 10, 4)), r.standard_normal((1, 10, 4))
    kv = DraftKV(1, 10, 4, Kp, Vp, length=5)
    out = hd.step(kv, 3, r.standard_normal(8))
    mean_v = Vp[0, :5].sum(axis=0) / 6.0
    g = np.concatenate([mean_v, mean_v])
    assert np.allclose(out["g"][0], g, atol=1e-14)
    assert np.allclose(out["logits"][:8], H.rmsnorm(g, np.ones(8), SMALL.rms_eps), atol=1e-13)
    assert np.all(out["logits"][8:] == 0)
    assert np.all(kv.K[0, 5] == 0) and np.all(kv.V[0, 5] == 0) and kv.len == 6


def test_concat_order_embedding_first():
    """fc = [I | 0] reads only the embedding half: g = x = RMSNorm(E[t]; w_pe),
    independent of the hidden; fc = [0 | I] reads only the hidden half."""
    w = zero_head()
    w["fc"][:, :8] = np.eye(8)
    w["pre_fc_norm_embedding"] = np.linspace(0.5, 2.0, 8).astype(np.float32)
    hd = H.Head(SMALL, w)
    r = np.random.default_rng(7)
    kv1, kv2 = DraftKV(1, 4, 4), DraftKV(1, 4, 4)
    a = hd.step(kv1, 9, r.standard_normal(8))
    b = hd.step(kv2, 9, 100 * r.standard_normal(8))
    e = w["embed"][9].astype(np.float64)
    want = e / math.sqrt(np.mean(e * e) + SMALL.rms_eps) * w["pre_fc_norm_embedding"]
    assert np.allclose(a["g"][0], want, atol=1e-14) and np.allclose(b["g"][0], want, atol=1e-14)
    w2 = zero_head()
    w2["fc"][:, 8:] = np.eye(8)
    hd2 = H.Head(SMALL, w2)
    h = r.standard_normal(8)
    c = hd2.step(DraftKV(1, 4, 4), 9, h)
    d = hd2.step(DraftKV(1, 4, 4), 2, h)
    assert np.allclose(c["g"][0], d["g"][0], atol=1e-15)
    assert np.allclose(c["g"][0], h / math.sqrt(np.mean(h * h) + SMALL.rms_eps), atol=1e-14)


def test_mlp_residual_identity_weights():
    """fc = [I|0], o_proj = 0, gate = up = down = I: g = x + silu(b) * b with
    b = RMSNorm(x; w_post)."""
    w = zero_head()
    w["fc"][:, :8] = np.eye(8)
    w["gate_proj"] = np.eye(8, dtype=np.float32)
    w["up_proj"] = np.eye(8, dtype=np.float32)
    w["down_proj"] = np.eye(8, dtype=np.float32)
    w["post_attention_layernorm"] = np.full(8, 2.0, np.float32)
    hd = H.Head(SMALL, w)
    out = hd.step(DraftKV(1, 4, 4), 4, np.ones(8))
    e = w["embed"][4].astype(np.float64)
    x = e / math.sqrt(np.mean(e * e) + SMALL.rms_eps)
    b = 2.0 * x / math.sqrt(np.mean(x * x) + SMALL.rms_eps)
    assert np.allclose(out["g"][0], x + b * b / (1 + np.exp(-b)), atol=1e-13)


def test_single_key_attention_returns_value():
    """At slot 0 with an empty cache the only key is the new one: o = v for every
    query head regardless of q; with o_proj = I, v_proj = [I_4 | 0] and fc = [I|0]
    we get g = x + [v, v] with v = RMSNorm(x; w_in)[:4]."""
    w = zero_head()
    w["fc"][:, :8] = np.eye(8)
    w["o_proj"] = np.eye(8, dtype=np.float32)
    w["v_proj"][:, :4] = np.eye(4)
    w["q_proj"] = np.random.default_rng(8).standard_normal((8, 8)).astype(np.float32)
    w["k_proj"] = np.random.default_rng(9).standard_normal((4, 8)).astype(np.float32)
    hd = H.Head(SMALL, w)
    out = hd.step(DraftKV(1, 4, 4), 11, np.zeros(8))
    e = w["embed"][11].astype(np.float64)
    x = e / math.sqrt(np.mean(e * e) + SMALL.rms_eps)
    a = x / math.sqrt(np.mean(x * x) + SMALL.rms_eps)
    assert np.allclose(out["g"][0], x + np.concatenate([a[:4], a[:4]]), atol=1e-13)


def test_qk_norm_before_rope():
    """Per-head RMSNorm comes before RoPE: the rotation-invariant pair norms of q
    and k are then the same at every position even with a non-uniform norm weight."""
    s = I.TINY_F32
    vals = I.weight_values(s, I.head_weights(s, 90))
    vals["q_norm"] = np.linspace(0.2, 3.0, s.head_dim).astype(np.float32)
    vals["k_norm"] = np.linspace(3.0, 0.2, s.head_dim).astype(np.float32)
    hd = H.Head(s, vals)
    x = hd.fused_input(5, np.random.default_rng(10).standard_normal(s.hidden))
    h2 = s.head_dim // 2
    q0, k0, v0 = hd.qkv(x, 0)
    q1, k1, v1 = hd.qkv(x, 777)
    for a, b in ((q0, q1), (k0, k1)):
        assert np.allclose(a[:, :h2] ** 2 + a[:, h2:] ** 2, b[:, :h2] ** 2 + b[:, h2:] ** 2, atol=1e-11)
    assert np.array_equal(v0, v1)
    # and at position 0 RoPE is the identity, so q is exactly the normed projection
    assert np.allclose(np.sqrt(np.mean((q0 / vals["q_norm"]) ** 2, axis=1)), 1.0, atol=1e-5)


def test_slot_is_the_rope_position():
    """A pair flushed at slot S is roped at position S: the score between a key
    written at slot S and a query at slot S + 1 is the same for S = 0 and S = 40."""
    s = I.TINY_F32
    hd = H.Head(s, I.weight_values(s, I.head_weights(s, 91)))
    r = np.random.default_rng(11)
    h, h2 = r.standard_normal(s.hidden), r.standard_normal(s.hidden)
    kvA, kvB = DraftKV(2, 64, 64), DraftKV(2, 64, 64, length=40)
    hd.flush(kvA, [7], [h], H.KV_ONLY)
    hd.flush(kvB, [7], [h], H.KV_ONLY)
    assert not np.allclose(kvA.K[:, 0], kvB.K[:, 40])          # the keys differ ...
    x = hd.fused_input(9, h2)
    qa, _, _ = hd.qkv(x, 1)
    qb, _, _ = hd.qkv(x, 41)
    for hq in range(4):
        kh = hq // 2
        assert abs(qa[hq] @ kvA.K[kh, 0] - qb[hq] @ kvB.K[kh, 40]) < 1e-10   # ... the scores do not


def test_block_equals_chain():
    """Flushing n pairs at once (ALL) equals n single-pair steps: every row's g,
    the K/V written, and the last row's logits."""
    s = I.TINY_F32
    vals = I.weight_values(s, I.head_weights(s, 92))
    hd = H.Head(s, vals)
    kp, vp = I.prefix_kv(s, 92, 16, 64)
    r = np.random.default_rng(12)
    toks = [int(t) for t in r.integers(0, s.vocab, 5)]
    hids = [r.standard_normal(s.hidden) for _ in range(5)]
    kv1 = DraftKV(2, 64, 64, kp, vp, 16)
    blk = hd.flush(kv1, toks, hids, H.ALL)
    kv2 = DraftKV(2, 64, 64, kp, vp, 16)
    rows = [hd.step(kv2, t, h) for t, h in zip(toks, hids)]
    for j in range(5):
        assert np.allclose(blk["g"][j], rows[j]["g"][0], atol=1e-12)
    assert np.allclose(blk["logits"], rows[-1]["logits"], atol=1e-12)
    assert np.array_equal(kv1.K, kv2.K) and np.array_equal(kv1.V, kv2.V)
    assert kv1.len == kv2.len == 21
    # LAST gives the same last row; KV_ONLY writes the same K/V
    kv3 = DraftKV(2, 64, 64, kp, vp, 16)
    last = hd.flush(kv3, toks, hids, H.LAST)
    assert np.allclose(last["g"][0], blk["g"][-1], atol=1e-13) and last["argmax"] == blk["argmax"]
    kv4 = DraftKV(2, 64, 64, kp, vp, 16)
    assert hd.flush(kv4, toks, hids, H.KV_ONLY) == {}
    assert np.array_equal(kv4.K, kv1.K)


def test_capacity_error_is_sticky():
    s = I.TINY_F32
    hd = H.Head(s, I.weight_values(s, I.head_weights(s, 93)))
    kv = DraftKV(2, 4, 64, length=3)
    assert hd.flush(kv, [1, 2], [np.zeros(256)] * 2, H.LAST) == {}
    assert kv.err != 0 and kv.len == 3
    assert hd.step(kv, 1, np.zeros(256)) == {}


def test_unbound_head_rejected():
    s = I.TINY_F32
    vals = I.weight_values(s, I.head_weights(s, 94))
    vals["lm_head"] = None
    with pytest.raises(ValueError):
        H.Head(s, vals)


def test_int8_lm_head_equals_dequantised_fp():
    """The int8 lm_head path equals the fp lm_head path on the dequantised values."""
    s = I.TINY_BF16.with_dtypes(lm_head_dtype=I.I8G128)
    st = I.head_weights(s, 95)
    vals = I.weight_values(s, st)
    hd = H.Head(s, vals)
    vals2 = dict(vals)
    vals2.pop("lm_head_scales")
    vals2["lm_head"] = (st["lm_head"].astype(np.float64).reshape(s.vocab, 2, 128)
                        * st["lm_head_scales"].astype(np.float64)[:, :, None]).reshape(s.vocab, 256)
    hd2 = H.Head(s.with_dtypes(lm_head_dtype=I.BF16), vals2)
    g = np.random.default_rng(13).standard_normal(256)
    assert np.allclose(hd.unembed(g), hd2.unembed(g), atol=1e-12)
