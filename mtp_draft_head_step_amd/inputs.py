"""Seeded synthetic inputs for the MTP draft round (head weights, draft KV prefix,
target hiddens and logits, uniforms, history rings).

This module holds no arithmetic of the method itself: it only draws numbers and
stores them in the layouts the library and the oracle both consume.  Every draw
uses ``numpy.random.default_rng([config_id, stream, tensor, chunk])`` so that
any tensor (or any chunk of a large tensor) can be regenerated on its own.

Streams: 0 projection weights, 1 norm weights, 2 embedding and lm_head,
3 prefix KV, 4 target hiddens, 5 target logits, 6 draft logits, 7 accept and
sample uniforms, 8 token ids and history, 9 spike positions, 10 draft-token
uniforms, 11 acceptance draws.

Notation N(a, b) in the workload descriptions is read as mean a and standard
deviation b.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

# --------------------------------------------------------------------------
# dtypes and bf16 storage
# --------------------------------------------------------------------------
F32, BF16, I8G128 = "f32", "bf16", "i8g128"
DTYPE_CODES = {F32: 0, BF16: 1, I8G128: 2}
QGROUP = 128  # columns per int8 quantisation group


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32 (large arrays are
    widened in chunks on a thread pool)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    flat = b.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint32)
    step = 1 << 22

    def work(i):
        np.left_shift(flat[i:i + step], 16, out=out[i:i + step], dtype=np.uint32)

    if flat.size <= step:
        work(0)
    else:
        with _cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(work, range(0, flat.size, step)))
    return out.view(np.float32).reshape(b.shape)


def decode(storage: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> fp32 values (exact)."""
    if dtype == BF16:
        return bf16_bits_to_f32(storage)
    if dtype == F32:
        return np.ascontiguousarray(storage, dtype=np.float32)
    raise ValueError(f"decode: unsupported dtype {dtype}")


def encode(values: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> storage in ``dtype`` (bf16 rounds to nearest even)."""
    if dtype == BF16:
        return f32_to_bf16_bits(values)
    if dtype == F32:
        return np.ascontiguousarray(values, dtype=np.float32)
    raise ValueError(f"encode: unsupported dtype {dtype}")


def quantize_i8g128(w: np.ndarray):
    """Symmetric per-(row, 128-column group) int8 quantisation with fp16 scales.

    s = fp16(absmax / 127) (round to nearest even), q = clamp(rint(w / s), -127, 127),
    and a group whose scale is 0 stores q = 0.  The dequantised weight is q * s.
    Returns (q int8 [M, K], s float16 [M, K/128]).
    """
    w = np.asarray(w, dtype=np.float32)
    m, k = w.shape
    if k % QGROUP:
        raise ValueError("quantize_i8g128: columns must be a multiple of 128")
    g = w.reshape(m, k // QGROUP, QGROUP)
    s16 = (np.abs(g).max(axis=2) / np.float32(127.0)).astype(np.float16)
    s = s16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8).reshape(m, k)
    return q, s16


# --------------------------------------------------------------------------
# head shapes and workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class HeadShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    weight_dtype: str = F32     # projections, norms and the embedding table
    act_dtype: str = F32        # hidden states crossing the boundary
    kv_dtype: str = F32         # draft KV cache
    lm_head_dtype: str = F32    # f32 | bf16 | i8g128

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_dtypes(self, **kw) -> "HeadShape":
        return dataclasses.replace(self, **kw)

    def head_param_count(self) -> int:
        h, i = self.hidden, self.intermediate
        return (2 * h * h                      # fc
                + (self.q_dim + 2 * self.kv_dim) * h
                + h * self.q_dim               # o_proj
                + 3 * h * i                    # gate, up, down
                + 5 * h + 2 * self.head_dim)   # norms


# Tiny head, fp32 throughout.
TINY_F32 = HeadShape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                     intermediate=768, vocab=1024)
# The same tiny head with bf16 weights, activations and KV.
TINY_BF16 = TINY_F32.with_dtypes(weight_dtype=BF16, act_dtype=BF16, kv_dtype=BF16,
                                 lm_head_dtype=BF16)
# Qwen3.5-27B-shaped MTP head: bf16 weights and activations, fp32 accumulate.
QWEN35_27B = HeadShape(hidden=5120, n_q_heads=24, n_kv_heads=4, head_dim=256,
                       intermediate=17408, vocab=152064, weight_dtype=BF16,
                       act_dtype=BF16, kv_dtype=BF16, lm_head_dtype=BF16)

# Workload ids used as the first seed word.
WL_TINY, WL_QWEN, WL_FLUSH, WL_VERIFY, WL_DEPTH = 1, 2, 3, 4, 5

HEAD_TENSORS = ("pre_fc_norm_embedding", "pre_fc_norm_hidden", "fc", "input_layernorm",
                "q_proj", "k_proj", "v_proj", "q_norm", "k_norm", "o_proj",
                "post_attention_layernorm", "gate_proj", "up_proj", "down_proj", "norm")
NORM_TENSORS = ("pre_fc_norm_embedding", "pre_fc_norm_hidden", "input_layernorm",
                "q_norm", "k_norm", "post_attention_layernorm", "norm")


def tensor_shapes(s: HeadShape) -> dict:
    h, d, i = s.hidden, s.head_dim, s.intermediate
    return {
        "pre_fc_norm_embedding": (h,), "pre_fc_norm_hidden": (h,), "fc": (h, 2 * h),
        "input_layernorm": (h,), "q_proj": (s.q_dim, h), "k_proj": (s.kv_dim, h),
        "v_proj": (s.kv_dim, h), "q_norm": (d,), "k_norm": (d,), "o_proj": (h, s.q_dim),
        "post_attention_layernorm": (h,), "gate_proj": (i, h), "up_proj": (i, h),
        "down_proj": (h, i), "norm": (h,), "embed": (s.vocab, h), "lm_head": (s.vocab, h),
    }


# --------------------------------------------------------------------------
# chunked, threaded normal draws
# --------------------------------------------------------------------------
_CHUNK = 1 << 22


def _normal_chunk(seed_words, n, mean, std):
    r = np.random.default_rng(list(seed_words))
    x = r.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def normal(seed_words, shape, mean=0.0, std=1.0, dtype=F32) -> np.ndarray:
    """N(mean, std) draws of ``shape``, chunked by 4M elements (each chunk has
    its own seed), stored in ``dtype`` (bf16 as uint16 bits)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)

    def work(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        x = _normal_chunk(tuple(seed_words) + (c,), hi - lo, mean, std)
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == BF16 else x

    if nchunks == 1:
        work(0)
    else:
        workers = min(16, os.cpu_count() or 1, nchunks)
        with _cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def head_weights(s: HeadShape, wl: int) -> dict:
    """The 15 head tensors plus the borrowed embedding table and lm_head.

    Projections and the embedding/lm_head are N(0, 0.02); norm weights are
    1 + N(0, 0.01).  Storage follows ``weight_dtype`` (the lm_head follows
    ``lm_head_dtype``; int8 adds ``lm_head_scales``).
    """
    shapes = tensor_shapes(s)
    out = {}
    for t, name in enumerate(HEAD_TENSORS):
        if name in NORM_TENSORS:
            out[name] = normal((wl, 1, t), shapes[name], 1.0, 0.01, s.weight_dtype)
        else:
            out[name] = normal((wl, 0, t), shapes[name], 0.0, 0.02, s.weight_dtype)
    out["embed"] = normal((wl, 2, 0), shapes["embed"], 0.0, 0.02, s.weight_dtype)
    if s.lm_head_dtype == I8G128:
        w = normal((wl, 2, 1), shapes["lm_head"], 0.0, 0.02, BF16)
        q, sc = quantize_i8g128(bf16_bits_to_f32(w))
        out["lm_head"], out["lm_head_scales"] = q, sc
    else:
        out["lm_head"] = normal((wl, 2, 1), shapes["lm_head"], 0.0, 0.02, s.lm_head_dtype)
    return out


def weight_values(s: HeadShape, w: dict) -> dict:
    """fp32 values of every stored bf16/f32 tensor; an int8 lm_head is passed
    through as (``lm_head`` int8, ``lm_head_scales`` fp16) storage."""
    v = {}
    for name, arr in w.items():
        if name in ("lm_head", "lm_head_scales") and s.lm_head_dtype == I8G128:
            v[name] = arr
        elif name == "lm_head":
            v[name] = decode(arr, s.lm_head_dtype)
        else:
            v[name] = decode(arr, s.weight_dtype)
    return v


def prefix_kv(s: HeadShape, wl: int, length: int, capacity: int):
    """Draft KV cache [n_kv_heads, capacity, head_dim] with slots [0, length)
    drawn N(0, 1) (stored in ``kv_dtype``) and the rest zero."""
    if length > capacity:
        raise ValueError("prefix longer than capacity")
    shape = (s.n_kv_heads, capacity, s.head_dim)
    st = np.uint16 if s.kv_dtype == BF16 else np.float32
    k = np.zeros(shape, dtype=st)
    v = np.zeros(shape, dtype=st)
    if length:
        k[:, :length] = normal((wl, 3, 0, length), (s.n_kv_heads, length, s.head_dim), 0, 1, s.kv_dtype)
        v[:, :length] = normal((wl, 3, 1, length), (s.n_kv_heads, length, s.head_dim), 0, 1, s.kv_dtype)
    return k, v


def target_hiddens(s: HeadShape, wl: int, key, rows: int) -> np.ndarray:
    """[rows, hidden] N(0, 1) target hidden states in ``act_dtype``; ``key``
    (an int or tuple) selects the round."""
    key = tuple(key) if isinstance(key, (tuple, list)) else (int(key),)
    return normal((wl, 4) + key, (rows, s.hidden), 0, 1, s.act_dtype)


def tokens_uniform(wl: int, key, n: int, vocab: int) -> np.ndarray:
    key = tuple(key) if isinstance(key, (tuple, list)) else (int(key),)
    return np.random.default_rng([wl, 8, *key]).integers(0, vocab, n).astype(np.int32)


def uniforms(wl: int, key, n: int, stream: int = 7) -> np.ndarray:
    """n fp32 uniforms in [0, 1)."""
    key = tuple(key) if isinstance(key, (tuple, list)) else (int(key),)
    return np.random.default_rng([wl, stream, *key]).random(n, dtype=np.float32)


def logits_rows(wl: int, stream: int, key, rows: int, vocab: int, std: float,
                spikes: int = 0, spike: float = 0.0, spike_positions=None):
    """[rows, vocab] fp32 N(0, std) logits; optionally ``spikes`` distinct
    positions per row get ``+spike`` (positions drawn on stream 9 unless given).
    Returns (logits, positions [rows, spikes])."""
    key = tuple(key) if isinstance(key, (tuple, list)) else (int(key),)
    x = normal((wl, stream) + key, (rows, vocab), 0.0, std, F32)
    pos = None
    if spikes:
        if spike_positions is None:
            r = np.random.default_rng([wl, 9, *key])
            pos = np.stack([r.choice(vocab, spikes, replace=False) for _ in range(rows)])
        else:
            pos = np.asarray(spike_positions)
        for i in range(rows):
            x[i, pos[i]] += np.float32(spike)
    return x, pos


def history_ring(wl: int, key, window: int, vocab: int):
    """A full ring of ``window`` uniform token ids (head 0, count window)."""
    key = 0 if key is None else key
    ring = tokens_uniform(wl, (77, key) if isinstance(key, int) else (77,) + tuple(key), window, vocab)
    return ring, np.array([0, window], dtype=np.int32)


def acceptance_draws(wl: int, key, n_draft: int, p0: float = 0.8, decay: float = 0.85):
    """Per-position Bernoulli draws with p_i = p0 * decay**i (0-based); returns
    the planted number of accepted drafts (first failure ends the run)."""
    key = tuple(key) if isinstance(key, (tuple, list)) else (int(key),)
    u = np.random.default_rng([wl, 11, *key]).random(n_draft)
    for i in range(n_draft):
        if u[i] >= p0 * decay ** i:
            return i
    return n_draft


# --------------------------------------------------------------------------
# a deterministic toy target (stand-in for the target model's forward)
# --------------------------------------------------------------------------
class ToyTarget:
    """Next-token logits and hidden state of a fake target, seeded by
    (position, previous token) only.  ``logits(prev, pos)`` is N(0, std) fp32 over
    the vocabulary; ``hidden(prev, pos)`` is N(0, 1) stored in ``act_dtype``.
    Because each row depends only on (prev, pos), the rows a verify forward sees
    along an accepted path are exactly the rows sequential decoding sees."""

    def __init__(self, wl: int, vocab: int, hidden: int, act_dtype: str = F32, std: float = 3.0,
                 follow: float = 0.0, spike: float = 12.0):
        self.wl, self.vocab, self.hidden, self.act_dtype, self.std = wl, vocab, hidden, act_dtype, std
        self.follow, self.spike = follow, spike

    def logits(self, prev: int, pos: int) -> np.ndarray:
        """N(0, std) row; with probability ``follow`` (a seeded coin per (prev, pos))
        token (prev + 1) mod V gets +spike, so the greedy next token is the successor."""
        r = np.random.default_rng([self.wl, 5, 1000003, int(pos), int(prev)])
        x = (r.standard_normal(self.vocab, dtype=np.float32) * np.float32(self.std)).astype(np.float32)
        if self.follow > 0.0 and r.random() < self.follow:
            x[(int(prev) + 1) % self.vocab] += np.float32(self.spike)
        return x

    def hidden_state(self, prev: int, pos: int) -> np.ndarray:
        r = np.random.default_rng([self.wl, 4, 1000003, int(pos), int(prev)])
        x = r.standard_normal(self.hidden, dtype=np.float32)
        return encode(x, self.act_dtype)

    def forward(self, tokens, start_pos: int):
        """Rows for tokens[j] processed at position start_pos + j:
        (logits [n, V] fp32, hiddens [n, H] in act_dtype)."""
        lg = np.stack([self.logits(t, start_pos + j) for j, t in enumerate(tokens)])
        hs = np.stack([self.hidden_state(t, start_pos + j) for j, t in enumerate(tokens)])
        return lg, hs


def plant_acceptance(rows, drafts, k: int, spike: float = 1000.0):
    """Make greedy verification accept exactly ``k`` drafts: target row i < N gets
    +spike at d_i when i < k and at (d_i + 1) mod V otherwise.  Works in place on a
    numpy array or a torch tensor (``drafts`` may live on the device; ``k`` is a
    host integer), so a round can be planted without reading the drafts back."""
    n = drafts.shape[0]
    v = rows.shape[1]
    for i in range(n):
        tok = drafts[i] if i < k else (drafts[i] + 1) % v
        rows[i, tok] += spike
    return rows
