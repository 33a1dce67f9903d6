"""The benchmark's algorithmic byte and flop counts (the numerators of every
roofline figure) against totals derived by hand from the workload shapes."""
import bench
from mtp_draft_head_step_amd import inputs as I


def test_27b_step_bytes():
    """Qwen3.5-27B-shaped head at KV length 4097: 786,484,224 B of head weights,
    1,557,135,360 B of bf16 lm_head, 16,781,312 B of K/V (2 x 4 heads x 256 x
    2 B x 4097), one 10,240 B embedding row, 20,480 B of hidden in/out."""
    s = I.QWEN35_27B
    assert s.head_param_count() * 2 == 786_484_224
    assert bench.step_bytes(s, 4097) == 786_484_224 + 1_557_135_360 + 16_781_312 + 10_240 + 20_480
    # logits written: + V x 4 B
    assert bench.step_bytes(s, 4097, with_logits=True) - bench.step_bytes(s, 4097) == 152_064 * 4


def test_27b_unembedding_bytes_bf16_and_int8():
    s = I.QWEN35_27B
    assert bench.unembed_bytes(s) == 152_064 * 5120 * 2 + 5120 * 4 + 5120 * 2
    q = s.with_dtypes(lm_head_dtype=I.I8G128)
    # int8 weights + one fp16 scale per 128 columns
    assert bench.unembed_bytes(q) == 152_064 * 5120 + 152_064 * 40 * 2 + 5120 * 4 + 5120 * 2


def test_tiny_flush256_flops():
    """The 256-pair ALL flush of the tiny head after 8192 slots: projections
    2 x 917,504 x 256 flop + the last row's unembedding 2 x 1024 x 256, causal
    attention 4 x 64 x 4 x sum_{i<256}(8193 + i) = 2,181,169,152 flop."""
    s = I.TINY_BF16
    assert bench.flush_attention_flops(s, 8192, 256) == 2_181_169_152
    assert bench.flush_projection_flops(s, 256, 256) == 2 * 917_504 * 256 + 2 * 1024 * 256


def test_27b_flush256_flops():
    """At the 27B shape: every projection of the head (fc, q/k/v, o, gate, up,
    down) for 256 rows, 2 flop per weight, plus the last row's unembedding;
    row j attends over 4096 + j + 1 keys."""
    s = I.QWEN35_27B
    per_row = 2 * 5120 * 5120 + (24 + 8) * 256 * 5120 + 24 * 256 * 5120 + 3 * 5120 * 17408
    assert bench.flush_projection_flops(s, 256, 256) == 2 * (256 * per_row + 152_064 * 5120)
    keys = 256 * 4097 + 256 * 255 // 2
    assert bench.flush_attention_flops(s, 4096, 256) == 4 * 256 * 24 * keys


def test_attention_bytes():
    s = I.QWEN35_27B
    # K and V of 4097 slots for 4 kv heads of 256 bf16, plus the fp32 roped q in and o out
    assert bench.attention_bytes(s, 4097) == 2 * 4 * 256 * 2 * 4097 + 2 * 24 * 256 * 4
