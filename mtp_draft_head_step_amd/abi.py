"""Thin ctypes binding of libmtp (include/mtp.h): the same entry points, with
argument marshalling only (torch tensors -> device pointers, the current HIP
stream).  Every computation runs in the library's kernels.  Importing this
module loads libmtp.so from the package directory and raises if it is missing:
there is no fallback path.

Small helpers own device memory for callers (torch allocations): ``Head`` keeps
the weight tensors alive next to the native head handle, ``DraftKV`` holds the
cache and its state words, ``Workspace`` a zero-initialised scratch buffer.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmtp.so")

MTP_OK, MTP_E_INVALID_ARG, MTP_E_UNSUPPORTED, MTP_E_NOT_BOUND = 0, -1, -2, -3
MTP_E_CAPACITY, MTP_E_HIP, MTP_E_DEVICE, MTP_E_WORKSPACE = -4, -5, -6, -7
MTP_F32, MTP_BF16, MTP_I8G128 = 0, 1, 2
KV_ONLY, LAST, ALL = 0, 1, 2
TO_ROUND_BASE = -1
DEV_OK, DEV_CAPACITY, DEV_ROLLBACK, DEV_COUNT, DEV_TOKEN = 0, 1, 2, 3, 4

WEIGHT_FIELDS = ("embed", "lm_head", "lm_head_scales", "pre_fc_norm_embedding",
                 "pre_fc_norm_hidden", "fc", "input_layernorm", "q_proj", "k_proj", "v_proj",
                 "q_norm", "k_norm", "o_proj", "post_attention_layernorm", "gate_proj",
                 "up_proj", "down_proj", "norm")

EXPORTS = ("mtp_status_string", "mtp_last_error", "mtp_head_create", "mtp_head_destroy", "mtp_workspace_bytes",
           "mtp_workspace_init", "mtp_draft_step", "mtp_draft_step_static", "mtp_flush_pairs", "mtp_draft_chain", "mtp_repair_pending",
           "spec_verify_workspace_bytes", "spec_verify", "spec_verify_rollback", "kv_rollback", "mtp_timing_begin",
           "mtp_timing_pause", "mtp_timing_elapsed", "mtp_timing_end", "mtp_depth_ctl_create",
           "mtp_batch_workspace_bytes", "mtp_draft_chain_batch", "spec_verify_batch", "kv_rollback_batch",
           "mtp_repair_pending_batch",
           "mtp_depth_ctl_destroy", "mtp_depth_ctl_next", "mtp_depth_ctl_report", "mtp_depth_ctl_state")


class mtp_head_config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("intermediate", C.c_int32), ("vocab", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("weight_dtype", C.c_int32), ("act_dtype", C.c_int32), ("kv_dtype", C.c_int32),
                ("lm_head_dtype", C.c_int32)]


class mtp_head_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_FIELDS]


class mtp_kv(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("capacity", C.c_int32), ("state", C.c_void_p)]


class spec_sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("repeat_penalty", C.c_float), ("top_p", C.c_float),
                ("min_p", C.c_float), ("top_k", C.c_int32), ("window", C.c_int32)]


def _load():
    # torch ships its own HIP runtime under the same soname; loading torch first
    # makes libmtp bind to that one copy, so both share one runtime and device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmtp.so is not built ({LIB_PATH}); run python -m mtp_draft_head_step_amd.build")
    lib = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    lib.mtp_status_string.restype = C.c_char_p
    lib.mtp_status_string.argtypes = [C.c_int]
    lib.mtp_last_error.restype = C.c_char_p
    lib.mtp_last_error.argtypes = []
    lib.mtp_head_create.restype = C.c_int
    lib.mtp_head_create.argtypes = [C.POINTER(mtp_head_config), C.POINTER(mtp_head_weights), C.POINTER(vp)]
    lib.mtp_head_destroy.restype = None
    lib.mtp_head_destroy.argtypes = [vp]
    lib.mtp_workspace_bytes.restype = sz
    lib.mtp_workspace_bytes.argtypes = [C.POINTER(mtp_head_config), i32, i32]
    lib.mtp_workspace_init.restype = C.c_int
    lib.mtp_workspace_init.argtypes = [vp, sz, vp]
    lib.mtp_draft_step.restype = C.c_int
    lib.mtp_draft_step.argtypes = [vp, C.POINTER(mtp_kv), vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mtp_draft_step_static.restype = C.c_int
    lib.mtp_draft_step_static.argtypes = [vp, C.POINTER(mtp_kv), vp, vp, vp, vp, vp, vp]
    lib.mtp_flush_pairs.restype = C.c_int
    lib.mtp_flush_pairs.argtypes = [vp, C.POINTER(mtp_kv), vp, vp, i32, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.mtp_draft_chain.restype = C.c_int
    lib.mtp_draft_chain.argtypes = [vp, C.POINTER(mtp_kv), vp, vp, i32, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.mtp_repair_pending.restype = C.c_int
    lib.mtp_repair_pending.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.spec_verify_workspace_bytes.restype = sz
    lib.spec_verify_workspace_bytes.argtypes = [i32, i32]
    lib.spec_verify.restype = C.c_int
    lib.spec_verify.argtypes = [C.POINTER(spec_sampling), i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mtp_batch_workspace_bytes.restype = sz
    lib.mtp_batch_workspace_bytes.argtypes = [C.POINTER(mtp_head_config), i32, i32, i32]
    lib.mtp_draft_chain_batch.restype = C.c_int
    lib.mtp_draft_chain_batch.argtypes = [vp, C.POINTER(mtp_kv), i32, vp, vp, i32, vp, i32, i32, vp, vp, vp, vp,
                                          sz, vp]
    lib.spec_verify_rollback.restype = C.c_int
    lib.spec_verify_rollback.argtypes = [C.POINTER(spec_sampling), i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                         C.POINTER(mtp_kv), i32, i32, vp, vp]
    lib.spec_verify_batch.restype = C.c_int
    lib.spec_verify_batch.argtypes = [C.POINTER(spec_sampling), i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      sz, vp]
    lib.kv_rollback_batch.restype = C.c_int
    lib.kv_rollback_batch.argtypes = [C.POINTER(mtp_kv), i32, i32, vp, i32, vp]
    lib.mtp_repair_pending_batch.restype = C.c_int
    lib.mtp_repair_pending_batch.argtypes = [i32, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.kv_rollback.restype = C.c_int
    lib.kv_rollback.argtypes = [C.POINTER(mtp_kv), i32, vp, i32, vp]
    lib.mtp_timing_begin.restype = C.c_int
    lib.mtp_timing_begin.argtypes = [i32, i32]
    lib.mtp_timing_pause.restype = C.c_int
    lib.mtp_timing_pause.argtypes = [i32]
    lib.mtp_timing_elapsed.restype = C.c_int
    lib.mtp_timing_elapsed.argtypes = [i32, i32, C.POINTER(C.c_float)]
    lib.mtp_timing_end.restype = C.c_int
    lib.mtp_timing_end.argtypes = [C.POINTER(C.c_float), C.POINTER(i32)]
    lib.mtp_depth_ctl_create.restype = C.c_int
    lib.mtp_depth_ctl_create.argtypes = [i32, C.POINTER(C.c_double), C.POINTER(vp)]
    lib.mtp_depth_ctl_destroy.restype = None
    lib.mtp_depth_ctl_destroy.argtypes = [vp]
    lib.mtp_depth_ctl_next.restype = i32
    lib.mtp_depth_ctl_next.argtypes = [vp]
    lib.mtp_depth_ctl_report.restype = C.c_int
    lib.mtp_depth_ctl_report.argtypes = [vp, i32, i32, C.c_double]
    lib.mtp_depth_ctl_state.restype = C.c_int
    lib.mtp_depth_ctl_state.argtypes = [vp, C.POINTER(i32), C.POINTER(i32), C.POINTER(C.c_double)]
    return lib


lib = _load()


class MtpError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = f"{where}: {lib.mtp_status_string(status).decode()} ({status})"
        if status == MTP_E_HIP:
            msg += f": {lib.mtp_last_error().decode()}"
        super().__init__(msg)


def _check(status, where):
    if status != MTP_OK:
        raise MtpError(status, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------
def mtp_status_string(status: int) -> str:
    return lib.mtp_status_string(status).decode()


def mtp_last_error() -> str:
    return lib.mtp_last_error().decode()


def mtp_head_create(cfg: mtp_head_config, weights: mtp_head_weights):
    h = C.c_void_p()
    st = lib.mtp_head_create(C.byref(cfg), C.byref(weights), C.byref(h))
    _check(st, "mtp_head_create")
    return h


def mtp_head_destroy(handle):
    lib.mtp_head_destroy(handle)


def mtp_workspace_bytes(cfg: mtp_head_config, max_rows: int, max_capacity: int) -> int:
    return lib.mtp_workspace_bytes(C.byref(cfg), max_rows, max_capacity)


def mtp_workspace_init(ws, nbytes: int, stream=None):
    _check(lib.mtp_workspace_init(_ptr(ws), nbytes, _stream(stream)), "mtp_workspace_init")


def mtp_draft_step(head, kv, token, hidden_in, hidden_out, logits, argmax, ws, stream=None):
    st = lib.mtp_draft_step(head.handle, C.byref(kv.desc), _ptr(token), _ptr(hidden_in),
                            _ptr(hidden_out), _ptr(logits), _ptr(argmax), _ptr(ws), ws.nbytes,
                            _stream(stream))
    _check(st, "mtp_draft_step")


def mtp_draft_step_static(head, kv, token, hidden_in, hidden_out, logits, argmax, stream=None):
    st = lib.mtp_draft_step_static(head.handle, C.byref(kv.desc), _ptr(token), _ptr(hidden_in),
                                   _ptr(hidden_out), _ptr(logits), _ptr(argmax), _stream(stream))
    _check(st, "mtp_draft_step_static")


def mtp_flush_pairs(head, kv, tokens, hiddens, n_max, n_dev, out_mode, set_round_base,
                    hidden_out, logits_last, argmax_last, ws, stream=None):
    st = lib.mtp_flush_pairs(head.handle, C.byref(kv.desc), _ptr(tokens), _ptr(hiddens), int(n_max),
                             _ptr(n_dev), int(out_mode), int(set_round_base), _ptr(hidden_out),
                             _ptr(logits_last), _ptr(argmax_last), _ptr(ws), ws.nbytes, _stream(stream))
    _check(st, "mtp_flush_pairs")


def mtp_draft_chain(head, kv, pend_tokens, pend_hiddens, n_max, n_dev, n_draft, drafts, hiddens_out,
                    draft_logits, ws, stream=None):
    st = lib.mtp_draft_chain(head.handle, C.byref(kv.desc), _ptr(pend_tokens), _ptr(pend_hiddens), int(n_max),
                             _ptr(n_dev), int(n_draft), _ptr(drafts), _ptr(hiddens_out), _ptr(draft_logits),
                             _ptr(ws), ws.nbytes, _stream(stream))
    _check(st, "mtp_draft_chain")


def mtp_repair_pending(out_tokens, out_counts, target_hiddens, hidden, act_dtype, n_draft, pend_tokens,
                       pend_hiddens, pend_count, stream=None):
    st = lib.mtp_repair_pending(_ptr(out_tokens), _ptr(out_counts), _ptr(target_hiddens), int(hidden),
                                int(act_dtype), int(n_draft), _ptr(pend_tokens), _ptr(pend_hiddens),
                                _ptr(pend_count), _stream(stream))
    _check(st, "mtp_repair_pending")


def spec_verify_workspace_bytes(n_draft: int, vocab: int) -> int:
    return lib.spec_verify_workspace_bytes(n_draft, vocab)


def spec_verify(sp: spec_sampling, n_draft, vocab, target_logits, draft_logits, draft_tokens,
                history, history_state, uniforms, out_tokens, out_counts, ws, stream=None):
    st = lib.spec_verify(C.byref(sp), int(n_draft), int(vocab), _ptr(target_logits), _ptr(draft_logits),
                         _ptr(draft_tokens), _ptr(history), _ptr(history_state), _ptr(uniforms),
                         _ptr(out_tokens), _ptr(out_counts), _ptr(ws), ws.nbytes, _stream(stream))
    _check(st, "spec_verify")


def spec_verify_rollback(sp: spec_sampling, n_draft, vocab, target_logits, draft_logits, draft_tokens,
                         history, history_state, uniforms, out_tokens, out_counts, ws, kv, to_len,
                         keep_accepted=False, report=None, stream=None):
    """`report`: a device tensor, a raw address (host-coherent pinned memory) or None."""
    st = lib.spec_verify_rollback(C.byref(sp), int(n_draft), int(vocab), _ptr(target_logits), _ptr(draft_logits),
                                  _ptr(draft_tokens), _ptr(history), _ptr(history_state), _ptr(uniforms),
                                  _ptr(out_tokens), _ptr(out_counts), _ptr(ws), ws.nbytes, C.byref(kv.desc),
                                  int(to_len), int(bool(keep_accepted)), _ptr(report), _stream(stream))
    _check(st, "spec_verify_rollback")


def kv_rollback(kv, to_len, n_accepted=None, n_draft=0, stream=None):
    st = lib.kv_rollback(C.byref(kv.desc), int(to_len), _ptr(n_accepted), int(n_draft), _stream(stream))
    _check(st, "kv_rollback")


def mtp_batch_workspace_bytes(cfg: mtp_head_config, batch: int, max_rows: int, max_capacity: int) -> int:
    return lib.mtp_batch_workspace_bytes(C.byref(cfg), int(batch), int(max_rows), int(max_capacity))


def mtp_draft_chain_batch(head, kv, batch, pend_tokens, pend_hiddens, n_max, n_dev, n_dev_stride, n_draft, drafts,
                          hiddens_out, draft_logits, ws, stream=None):
    st = lib.mtp_draft_chain_batch(head.handle, C.byref(kv.desc), int(batch), _ptr(pend_tokens), _ptr(pend_hiddens),
                                   int(n_max), _ptr(n_dev), int(n_dev_stride), int(n_draft), _ptr(drafts),
                                   _ptr(hiddens_out), _ptr(draft_logits), _ptr(ws), ws.nbytes, _stream(stream))
    _check(st, "mtp_draft_chain_batch")


def spec_verify_batch(sp: spec_sampling, batch, n_draft, vocab, target_logits, draft_logits, draft_tokens,
                      history, history_state, uniforms, out_tokens, out_counts, ws, stream=None):
    st = lib.spec_verify_batch(C.byref(sp), int(batch), int(n_draft), int(vocab), _ptr(target_logits),
                               _ptr(draft_logits), _ptr(draft_tokens), _ptr(history), _ptr(history_state),
                               _ptr(uniforms), _ptr(out_tokens), _ptr(out_counts), _ptr(ws), ws.nbytes,
                               _stream(stream))
    _check(st, "spec_verify_batch")


def kv_rollback_batch(kv, batch, to_len, counts=None, n_draft=0, stream=None):
    st = lib.kv_rollback_batch(C.byref(kv.desc), int(batch), int(to_len), _ptr(counts), int(n_draft),
                               _stream(stream))
    _check(st, "kv_rollback_batch")


def mtp_repair_pending_batch(batch, out_tokens, out_counts, target_hiddens, hidden, act_dtype, n_draft, pend_tokens,
                             pend_hiddens, pend_counts, stream=None):
    st = lib.mtp_repair_pending_batch(int(batch), _ptr(out_tokens), _ptr(out_counts), _ptr(target_hiddens),
                                      int(hidden), int(act_dtype), int(n_draft), _ptr(pend_tokens),
                                      _ptr(pend_hiddens), _ptr(pend_counts), _stream(stream))
    _check(st, "mtp_repair_pending_batch")


TIME_UNEMBED, TIME_ATTENTION, TIME_VERIFY, TIME_PROJECTION = 0, 1, 2, 3


def mtp_timing_begin(kind: int, max_launches: int):
    """Time the next ``max_launches`` launches of kernel class ``kind``."""
    _check(lib.mtp_timing_begin(int(kind), int(max_launches)), "mtp_timing_begin")


def mtp_timing_pause(paused: bool):
    """Suspend or resume bracketing launches (the slots are kept)."""
    _check(lib.mtp_timing_pause(1 if paused else 0), "mtp_timing_pause")


def mtp_timing_elapsed(first: int, count: int) -> float:
    ms = C.c_float()
    _check(lib.mtp_timing_elapsed(int(first), int(count), C.byref(ms)), "mtp_timing_elapsed")
    return ms.value


def mtp_timing_end():
    """-> (summed kernel milliseconds of the timed class, launches timed)."""
    ms = C.c_float()
    n = C.c_int32()
    _check(lib.mtp_timing_end(C.byref(ms), C.byref(n)), "mtp_timing_end")
    return ms.value, n.value


class DepthController:
    """The library's draft-depth controller (host object): next() -> depth to
    draft this round; report(depth, accepted, round_cost) after the round."""

    def __init__(self, max_depth: int, cost):
        if max_depth < 0 or len(cost) != max_depth + 1:
            raise MtpError(MTP_E_INVALID_ARG, "mtp_depth_ctl_create")
        arr = (C.c_double * (max_depth + 1))(*[float(c) for c in cost])
        h = C.c_void_p()
        _check(lib.mtp_depth_ctl_create(max_depth, arr, C.byref(h)), "mtp_depth_ctl_create")
        self.max_depth = max_depth
        self.h = h

    def next(self) -> int:
        d = lib.mtp_depth_ctl_next(self.h)
        _check(min(d, 0), "mtp_depth_ctl_next")
        return d

    def report(self, depth: int, accepted: int, round_cost: float):
        _check(lib.mtp_depth_ctl_report(self.h, depth, accepted, float(round_cost)), "mtp_depth_ctl_report")

    def state(self):
        """-> (choice, probe interval, cost table)."""
        ch, iv = C.c_int32(), C.c_int32()
        cost = (C.c_double * (self.max_depth + 1))()
        _check(lib.mtp_depth_ctl_state(self.h, C.byref(ch), C.byref(iv), cost), "mtp_depth_ctl_state")
        return ch.value, iv.value, list(cost)

    def __del__(self):
        if getattr(self, "h", None):
            lib.mtp_depth_ctl_destroy(self.h)
            self.h = None


# ----------------------------------------------------------------------------
# owners of device memory (torch allocations)
# ----------------------------------------------------------------------------
def to_device(arr: np.ndarray, device="cuda"):
    """numpy storage -> torch device tensor (uint16 is bf16 bits, float16 stays)."""
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def config_of(shape) -> mtp_head_config:
    code = {"f32": MTP_F32, "bf16": MTP_BF16, "i8g128": MTP_I8G128}
    return mtp_head_config(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                           shape.intermediate, shape.vocab, shape.rms_eps, shape.rope_theta,
                           code[shape.weight_dtype], code[shape.act_dtype], code[shape.kv_dtype],
                           code[shape.lm_head_dtype])


class Head:
    """Weights on the device plus the native head handle."""

    def __init__(self, shape, storage: dict, device="cuda"):
        self.shape = shape
        self.cfg = config_of(shape)
        self.tensors = {k: to_device(v, device) for k, v in storage.items() if v is not None}
        w = mtp_head_weights()
        for name in WEIGHT_FIELDS:
            t = self.tensors.get(name)
            setattr(w, name, t.data_ptr() if t is not None else None)
        self.weights = w
        self.handle = mtp_head_create(self.cfg, w)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            mtp_head_destroy(h)
            self.handle = None


class DraftKV:
    """K, V [n_kv_heads, capacity, head_dim] and the state words {len, base, -, err}."""

    def __init__(self, shape, capacity: int, k=None, v=None, length: int = 0, device="cuda", state=None):
        """``state`` (optional): an int32 device tensor of 4 elements to hold the
        state words (for instance a slice of a buffer the caller copies back
        with other per-round results); it is initialised here."""
        import torch
        dt = torch.bfloat16 if shape.kv_dtype == "bf16" else torch.float32
        size = (shape.n_kv_heads, capacity, shape.head_dim)
        self.k = to_device(k, device) if k is not None else torch.zeros(size, dtype=dt, device=device)
        self.v = to_device(v, device) if v is not None else torch.zeros(size, dtype=dt, device=device)
        assert tuple(self.k.shape) == size and self.k.dtype == dt
        if state is None:
            self.state = torch.tensor([length, length, 0, 0], dtype=torch.int32, device=device)
        else:
            assert state.dtype == torch.int32 and state.numel() == 4 and state.is_contiguous()
            state.copy_(torch.tensor([length, length, 0, 0], dtype=torch.int32))
            self.state = state
        self.capacity = capacity
        self.desc = mtp_kv(self.k.data_ptr(), self.v.data_ptr(), capacity, self.state.data_ptr())


class BatchKV:
    """The draft KV of ``batch`` independent sessions in one allocation: K, V
    [batch, n_kv_heads, capacity, head_dim] and the state words [batch, 4]
    ({len, base, -, err} per session)."""

    def __init__(self, shape, batch: int, capacity: int, k=None, v=None, lengths=None, device="cuda"):
        import torch
        dt = torch.bfloat16 if shape.kv_dtype == "bf16" else torch.float32
        size = (batch, shape.n_kv_heads, capacity, shape.head_dim)
        self.k = to_device(k, device) if k is not None else torch.zeros(size, dtype=dt, device=device)
        self.v = to_device(v, device) if v is not None else torch.zeros(size, dtype=dt, device=device)
        assert tuple(self.k.shape) == size and self.k.dtype == dt
        lengths = [0] * batch if lengths is None else [int(x) for x in lengths]
        self.state = torch.tensor([[n, n, 0, 0] for n in lengths], dtype=torch.int32, device=device)
        self.batch, self.capacity = batch, capacity
        self.desc = mtp_kv(self.k.data_ptr(), self.v.data_ptr(), capacity, self.state.data_ptr())


class Workspace:
    def __init__(self, nbytes: int, device="cuda"):
        import torch
        if nbytes <= 0:
            raise MtpError(MTP_E_INVALID_ARG, "Workspace")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.nbytes = nbytes
        mtp_workspace_init(self.buf, nbytes)

    def data_ptr(self):
        return self.buf.data_ptr()


def sampling(temperature=0.0, repeat_penalty=1.0, top_k=0, top_p=1.0, min_p=0.0, window=64):
    return spec_sampling(temperature, repeat_penalty, top_p, min_p, top_k, window)
