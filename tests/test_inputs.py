"""The seeded input generators: bf16 rounding against torch's conversion, the
int8 quantiser's error bound, determinism, and the facts the pages print."""
import json
import os

import numpy as np
import torch

from mtp_draft_head_step_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def test_bf16_round_to_nearest_even_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0]   # exact ties
    ours = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(I.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic_and_chunk_seeded():
    a = I.normal((1, 2, 3), (3, 5000000), 0, 1, I.BF16)
    b = I.normal((1, 2, 3), (3, 5000000), 0, 1, I.BF16)
    assert np.array_equal(a, b)
    c = I.normal((1, 2, 4), (10,), 0, 1)
    assert not np.array_equal(a.reshape(-1)[:10], c)
    s = I.TINY_F32
    w = I.head_weights(s, 1)
    assert np.abs(w["fc"].std() - 0.02) < 0.002 and np.abs(w["norm"].mean() - 1.0) < 0.005


def test_quantizer_bound_and_zero_group():
    w = np.random.default_rng(1).standard_normal((16, 512)).astype(np.float32) * 0.02
    w[5, :128] = 0
    q, s = I.quantize_i8g128(w)
    assert q.dtype == np.int8 and s.dtype == np.float16 and s.shape == (16, 4)
    assert np.all(q[5, :128] == 0) and s[5, 0] == 0
    deq = q.astype(np.float64).reshape(16, 4, 128) * s.astype(np.float64)[:, :, None]
    err = np.abs(deq.reshape(16, 512) - w)
    assert np.all(err <= s.astype(np.float64).repeat(128, 1) * 0.5 + 1e-6)


def test_pages_facts():
    g = json.load(open(GOLDEN))
    names = {n.split(".")[-2] if "layers" not in n else n.split(".")[-2] for n in g["mtp_tensors"]}
    assert len(g["mtp_tensors"]) == 15 == len(I.HEAD_TENSORS)
    assert names == set(I.HEAD_TENSORS)
    norm_names = {sfx.strip(".").split(".")[0] for sfx in g["norm_offset_suffixes"]}
    assert norm_names == set(I.NORM_TENSORS)
    assert I.QWEN35_27B.hidden == g["hidden_size"] and I.QWEN35_27B.head_dim == g["head_dim"]
    assert g["block_size"] == g["mtp_depth"] + 2 and g["drafts_per_round"] == g["block_size"] - 1
    # 256 pending hiddens of 5120 bf16 values are exactly 2.5 MiB
    assert g["flush_cap_tokens"] * g["hidden_size"] * 2 == g["pinned_hidden_mib"] * 2 ** 20
