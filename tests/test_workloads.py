"""Shape and recipe checks of the seeded workload generators (CPU, no oracle arithmetic)."""
import numpy as np
import pytest

from block_sparse_gqa_paged_amd import workloads as W


def _check_paged(w):
    B, T, H, G, D = w["B"], w["T"], w["H"], w["G"], w["D"]
    assert w["cu"].shape == (B + 1,) and w["cu"][0] == 0 and w["cu"][-1] == T
    L = w["past"] + np.diff(w["cu"])
    need = (L + w["bs"] - 1) // w["bs"]
    assert need.max() <= w["MB"]
    bt = w["block_table"]
    live = np.concatenate([bt[b, :need[b]] for b in range(B)])
    assert (live >= 0).all() and (live < w["NB"]).all()
    assert len(np.unique(live)) == len(live)          # no block shared between sequences
    assert w["key_cache"].shape == (w["NB"], w["bs"], G, D)
    qs = (H + 2 * G) * D if w["packed"] else H * D
    assert w["query"].shape == (T, qs) and w["query"].dtype == np.float16
    return L


def test_tiny_decode():
    w = W.tiny_decode()
    L = _check_paged(w)
    assert list(w["past"]) == [37, 100] and list(w["cu"]) == [0, 1, 2]
    assert w["NB"] == 16 and sorted(w["block_table"].reshape(-1)) == list(range(16))
    assert list(L) == [38, 101] and w["scale"] == 0.125


@pytest.mark.parametrize("mode", [W.ROTARY_NEOX, W.ROTARY_INTERLEAVED])
def test_rotary_append_decode(mode):
    w = W.rotary_append_decode(rotary_mode=mode)
    _check_paged(w)
    assert w["cos"].shape == (4096, 64) and w["past"].max() < 4095
    pos = w["past"]
    bt = w["block_table"]
    assert np.array_equal(w["slot_mapping"],
                          bt[np.arange(4), pos // 32] * 32 + pos % 32)
    # the tables are cos/sin of pos * 10000^(-2i/128), rounded to fp16
    assert w["cos"][0].astype(np.float32).min() == 1.0 and not w["sin"][0].any()
    assert abs(float(w["sin"][1, 0]) - np.sin(1.0)) < 1e-3


def test_gqa_decode_recipe():
    w = W.gqa_decode(batch=8)          # same recipe, smaller batch to keep the test quick
    L = _check_paged(w)
    assert (w["past"] >= 512).all() and (w["past"] <= 8192).all()
    assert w["MB"] == 513
    need = int(((L + 15) // 16).sum())
    assert w["NB"] == int(np.ceil(1.1 * need))
    assert (w["block_table"] == -1).sum() == w["B"] * 513 - need


def test_sparse_recipe_statistics():
    sw = W.sparse_workload(4, Tq=256, hkv=8, qhead=4, head_dim=16, block_size=64, page_size=16,
                           batch=2, key_capacity=32768)
    E = sw["E"]
    assert sw["edge_meta"].shape == (E, 5)
    per_group = np.diff(sw["group_ptr"])
    # window of 4 + block 0 + 5% of the remaining ~507 blocks: ~30 per (q, h)
    assert 25 < per_group.mean() < 36
    em = sw["edge_meta"]
    key = (em[:, 0].astype(np.int64) * 8 + em[:, 1]) * 1024 + em[:, 2]
    assert np.all(np.diff(key) > 0)                      # sorted by (q_idx, h, blk), unique
    assert (em[:, 4] >= 0).all() and (em[:, 4] <= 64).all()
    assert np.isclose((sw["block_tables"] == -1).mean(), 0.10, atol=1e-3)
    # the last block of each batch is partial and kept by every query's window
    assert (em[:, 4] < 64).any()
