"""Helpers shared by the GPU parity tests: build the same seeded head for the HIP
path and the oracle, move results back, and apply the parity tolerances.

Tolerances: fp32 heads max|gpu - ref| <= 1e-4 * max|ref| per row or vector;
bf16 heads 2e-2 * max|ref| (the activation and KV roundings to bf16 plus fp32
accumulation order).  Integer results (tokens, counts, lengths) are exact.
"""
import numpy as np

from mtp_draft_head_step_amd import inputs as I

F32_TOL = 1e-4
BF16_TOL = 2e-2


def tol_of(shape):
    return BF16_TOL if shape.weight_dtype == I.BF16 or shape.act_dtype == I.BF16 or shape.kv_dtype == I.BF16 else F32_TOL


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def device_array(arr):
    from mtp_draft_head_step_amd import abi
    return abi.to_device(np.ascontiguousarray(arr))


def build(shape, wl):
    """(storage dict, GPU head, oracle head)."""
    from mtp_draft_head_step_amd import abi
    from oracle import head as OH
    st = I.head_weights(shape, wl)
    gh = abi.Head(shape, st)
    oh = OH.Head(shape, I.weight_values(shape, st))
    return st, gh, oh


def kv_pair(shape, wl, prefix, capacity):
    """A GPU DraftKV and an oracle DraftKV holding the same synthetic prefix."""
    from mtp_draft_head_step_amd import abi
    from oracle.kvcache import DraftKV
    kp, vp = I.prefix_kv(shape, wl, prefix, capacity)
    g = abi.DraftKV(shape, capacity, kp, vp, prefix)
    o = DraftKV(shape.n_kv_heads, capacity, shape.head_dim,
                I.decode(kp, shape.kv_dtype), I.decode(vp, shape.kv_dtype), prefix)
    return g, o


def argmax_ok(gpu_tok, ref_logits, gpu_logits):
    """The GPU argmax equals the oracle's, or the oracle's top-two margin is within
    twice the largest logit difference (a near tie, where both are correct)."""
    ref_tok = int(np.argmax(ref_logits))
    if int(gpu_tok) == ref_tok:
        return True, False
    bound = 2.0 * np.max(np.abs(np.asarray(gpu_logits, np.float64) - ref_logits))
    return bool(ref_logits[ref_tok] - ref_logits[int(gpu_tok)] <= bound), True
