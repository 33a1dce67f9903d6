"""Oracle: the MTP draft head (one full-attention decoder layer behind a fused
embedding/hidden projection), evaluated row by row in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes, for the pair stored at draft-KV slot S = (look-ahead token
t_{S+1}, target hidden h_S):

  xc     = [ RMSNorm(E[t_{S+1}]; w_pe) | RMSNorm(h_S; w_ph) ]          (embedding half first)
  x      = W_fc xc                                                     (2H -> H, no bias)
  a      = RMSNorm(x; w_in)
  q,k,v  = W_q a, W_k a, W_v a;  per-head RMSNorm of q and k over head_dim
  q,k    = RoPE(q, S), RoPE(k, S);  K[S], V[S] = k, v
  o_h    = softmax(q_h K[0..S]^T / sqrt(D)) V[0..S]   with kv head h // (Hq/Hkv)
  x1     = x + W_o o
  g      = x1 + W_down( silu(W_gate b) * (W_up b) ),  b = RMSNorm(x1; w_post)
  logits = W_lm RMSNorm(g; w_norm)                                    (borrowed lm_head)

Sources: "feat(inference): support the qwen3_5_mtp drafter ..." section
"Upstream contract to port" (module shape: fc 2H->H, the two pre-fc norms, the
layer list built as full attention, the final norm; the forward concatenating the
normed token embedding and the normed hidden before fc; embed_tokens and lm_head
borrowed from the target), section "Where the MTP weights actually live" (the 15
tensors: fc, norm, the two pre-fc norms, input/post-attention layernorms,
gate/up/down, q/k/v/o and q/k norms), and "Ollama qwen3_5 MTP loader and
SelfDraft path", Facts "MTP drafting" (slot S pairs the look-ahead token at S+1
with the target hidden at S; pending pairs flush in batches).

Readings where the pages are silent: RoPE is the rotate-half form over the whole
head_dim with angle S * theta^(-2i/D); q/k norms come before RoPE; GQA groups are
contiguous; the attention scale is 1/sqrt(D); the hidden fed to a chained step is
g (before the final norm); the lm_head may be int8 per (row, 128-column group)
with fp16 scales, dequantised as q * s.
"""
from __future__ import annotations

import numpy as np

KV_ONLY, LAST, ALL = 0, 1, 2
QGROUP = 128


def rmsnorm(x, w, eps):
    """x * (mean(x^2) + eps)^(-1/2) * w over the last axis, fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope(x, pos, theta):
    """Rotate-half RoPE at integer position ``pos`` over the last axis (length D):
    pairs (i, i + D/2) are rotated by the angle pos * theta^(-2i/D)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = float(pos) * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def matvec(w, x, rows_per_block=8192):
    """y = W x for W [M, K] (any float dtype) and x [..., K], in fp64.  Rows are
    taken in blocks only to bound memory; every output element is one fp64 dot
    product over the whole row."""
    x = np.asarray(x, dtype=np.float64)
    m = w.shape[0]
    out = np.empty(x.shape[:-1] + (m,), dtype=np.float64)
    for r0 in range(0, m, rows_per_block):
        r1 = min(m, r0 + rows_per_block)
        out[..., r0:r1] = x @ np.asarray(w[r0:r1], dtype=np.float64).T
    return out


def dequant_i8g128(q, s16):
    """int8 weights q [M, K] with fp16 scales s [M, K/128] -> fp64 q * s."""
    m, k = q.shape
    s = np.asarray(s16, dtype=np.float64)
    return (np.asarray(q, dtype=np.float64).reshape(m, k // QGROUP, QGROUP)
            * s[:, :, None]).reshape(m, k)


def attend(q, K, V, length):
    """Causal single-query attention for every query head.

    q [Hq, D]; K, V [Hkv, capacity, D]; keys 0..length-1 are visible.  Query head
    h reads kv head h // (Hq / Hkv).  Returns o [Hq, D]."""
    hq, d = q.shape
    group = hq // K.shape[0]
    o = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        kh = h // group
        s = (K[kh, :length] @ q[h]) / np.sqrt(d)
        p = np.exp(s - s.max())
        p /= p.sum()
        o[h] = p @ V[kh, :length]
    return o


class Head:
    """The draft head with its 15 tensors plus the borrowed embedding table and
    lm_head, all given as numpy arrays of their values (fp32 for f32/bf16
    storage; for an int8 lm_head, ``lm_head`` int8 and ``lm_head_scales`` fp16)."""

    def __init__(self, shape, values: dict, cache_fp64: bool = False):
        """``cache_fp64`` keeps an fp64 copy of every projection matrix (the same
        values; it only saves re-widening them at each product, for many-row
        flushes of large heads)."""
        self.s = shape
        self.w = dict(values)
        if values.get("embed") is None or values.get("lm_head") is None:
            raise ValueError("draft head is not bound to a target embedding/lm_head")
        self.group = shape.n_q_heads // shape.n_kv_heads
        if cache_fp64:
            for name in ("fc", "q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj"):
                self.w[name] = np.asarray(values[name], dtype=np.float64)

    # -- pieces -----------------------------------------------------------
    def fused_input(self, token, hidden):
        """x = W_fc [RMSNorm(E[token]; w_pe) | RMSNorm(hidden; w_ph)]."""
        w, eps = self.w, self.s.rms_eps
        e = np.asarray(w["embed"][int(token)], dtype=np.float64)
        xc = np.concatenate([rmsnorm(e, w["pre_fc_norm_embedding"], eps),
                             rmsnorm(hidden, w["pre_fc_norm_hidden"], eps)])
        return matvec(w["fc"], xc)

    def qkv(self, x, pos):
        """Attention inputs at slot ``pos``: q [Hq, D], k, v [Hkv, D] (q, k normed and roped)."""
        s, w = self.s, self.w
        a = rmsnorm(x, w["input_layernorm"], s.rms_eps)
        d = s.head_dim
        q = matvec(w["q_proj"], a).reshape(s.n_q_heads, d)
        k = matvec(w["k_proj"], a).reshape(s.n_kv_heads, d)
        v = matvec(w["v_proj"], a).reshape(s.n_kv_heads, d)
        q = rope(rmsnorm(q, w["q_norm"], s.rms_eps), pos, s.rope_theta)
        k = rope(rmsnorm(k, w["k_norm"], s.rms_eps), pos, s.rope_theta)
        return q, k, v

    def finish(self, x, o):
        """Residual o_proj and the SwiGLU MLP: returns g (the pre-final-norm output)."""
        w, eps = self.w, self.s.rms_eps
        x1 = x + matvec(w["o_proj"], o.reshape(-1))
        b = rmsnorm(x1, w["post_attention_layernorm"], eps)
        m = silu(matvec(w["gate_proj"], b)) * matvec(w["up_proj"], b)
        return x1 + matvec(w["down_proj"], m)

    def unembed(self, g):
        """logits = W_lm RMSNorm(g; w_norm) through the borrowed lm_head."""
        w = self.w
        n = rmsnorm(g, w["norm"], self.s.rms_eps)
        if "lm_head_scales" in w:
            lm = w["lm_head"]
            out = np.empty(lm.shape[0], dtype=np.float64)
            for r0 in range(0, lm.shape[0], 8192):
                r1 = min(lm.shape[0], r0 + 8192)
                out[r0:r1] = dequant_i8g128(lm[r0:r1], w["lm_head_scales"][r0:r1]) @ n
            return out
        return matvec(w["lm_head"], n)

    # -- the two entry points ---------------------------------------------
    def flush(self, kv, tokens, hiddens, mode=LAST, set_round_base=False, out_rows=None):
        """Pending-pair flush: n complete pairs (tokens[j], hiddens[j]) occupy
        slots kv.len + j.  Every row's K/V is written first (a pair's K/V depends
        only on that pair), then each requested row attends causally over
        [0, slot].  Modes: KV_ONLY (K/V only), LAST (the last row's g, logits and
        argmax), ALL (every row's g plus the last row's logits and argmax;
        ``out_rows`` may name a subset of the rows whose g is evaluated, for
        sampled comparisons of large flushes).  ``set_round_base`` records
        kv.base = kv.len after the append.

        Returns a dict with 'g' ([rows, H] fp64), 'logits' ([V] fp64) and
        'argmax' (int), or {} for KV_ONLY / a device-side error."""
        n = len(tokens)
        if n == 0:
            if set_round_base and not kv.err:
                kv.base = kv.len
            return {}
        off = kv.len
        if not kv.can_append(n):
            return {}
        xs, kvs = [], []
        for j in range(n):
            x = self.fused_input(tokens[j], hiddens[j])
            q, k, v = self.qkv(x, off + j)
            kv.write(off + j, k, v)
            xs.append(x)
            kvs.append(q)
        kv.len = off + n
        if set_round_base:
            kv.base = kv.len
        if mode == KV_ONLY:
            return {}
        rows = (range(n) if out_rows is None else sorted(out_rows)) if mode == ALL else [n - 1]
        g = np.stack([self.finish(xs[j], attend(kvs[j], kv.K, kv.V, off + j + 1)) for j in rows])
        last = g[-1] if rows[-1] == n - 1 else self.finish(xs[n - 1], attend(kvs[n - 1], kv.K, kv.V, off + n))
        logits = self.unembed(last)
        return {"g": g, "logits": logits, "argmax": int(np.argmax(logits))}

    def step(self, kv, token, hidden):
        """One draft-head step at slot kv.len: the flush of a single pair in LAST mode."""
        return self.flush(kv, [token], [hidden], LAST, False)
