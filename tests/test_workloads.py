"""The seeded input generator: reproducible, the stated shapes and structure."""
import numpy as np

import workloads


def test_tiny_is_reproducible_and_shaped():
    a = workloads.make_inputs(workloads.CONFIGS["tiny"])
    b = workloads.make_inputs(workloads.CONFIGS["tiny"])
    for key in ("q", "k", "w", "kv_fp4", "kv_scale", "block_table", "limit", "neg_slots"):
        assert np.array_equal(a[key], b[key]), key
    assert a["q"].shape == (1, 4, 64, 128) and a["q"].dtype == np.uint16
    assert a["k"].shape == (1, 256, 128)
    assert a["w"].shape == (1, 4, 64) and a["w"].dtype == np.float32
    assert list(a["limit"][0]) == [252, 253, 254, 255]
    assert a["kv_fp4"].shape == (4, 64, 64) and a["kv_scale"].shape == (4, 64, 4)
    assert sorted(a["block_table"][0].tolist()) == [0, 1, 2, 3]
    assert (a["kv_scale"] == 0xFF).sum() == 4
    other = a["kv_scale"][a["kv_scale"] != 0xFF]
    assert other.min() >= 120 and other.max() <= 134
    assert a["neg_slots"].shape == (4, 3)


def test_fp8_custom_scales_and_bytes():
    x = workloads.custom(B=1, T=3, K=70, topk=8, dtype="fp8", causal_offset=60)
    assert x["q"].dtype == np.uint8 and x["k"].dtype == np.uint8
    assert x["q_scale"].shape == (1, 3, 64) and x["k_scale"].shape == (1, 70)
    assert np.all(x["q_scale"] > 0) and np.all(x["k_scale"] > 0)
    # amax scaling: every (t,h) vector reaches +-448 (code 0x7E / 0xFE)
    assert np.all(np.any((x["q"] & 0x7F) == 0x7E, axis=-1))
    assert not np.any((x["q"] & 0x7F) == 0x7F)          # no NaN codes
    assert list(x["limit"][0]) == [60, 61, 62]


def test_decode_lengths_and_tables():
    cfg = workloads.Config("t", seed=9, B=5, T=1, K=1000, topk=8, len_range=(100, 1000))
    x = workloads.make_inputs(cfg)
    lens = x["seq_len"]
    assert np.all((lens >= 100) & (lens <= 1000))
    assert np.array_equal(x["limit"][:, 0], lens - 1)
    nblk = (lens + 63) // 64
    used = np.concatenate([x["block_table"][b, :nblk[b]] for b in range(5)])
    assert sorted(used.tolist()) == list(range(int(nblk.sum())))
    for b in range(5):                                   # keys past the length stay zero
        assert np.all(x["k"][b, lens[b]:] == 0)
