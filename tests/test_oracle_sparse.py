"""Pins of the oracle's block-sparse edge forward (alice-llm sparse_attention_forward.wgsl).

Merged over each (q_idx, h) group, the per-edge partials must equal dense softmax attention of
the query over the union of its edges' mapped keys; torch SDPA in float64 is the reference.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from block_sparse_gqa_paged_amd import workloads as W


def _sw(seed, all_blocks=False, unmapped=0.0, **kw):
    args = dict(Tq=12, hkv=2, qhead=2, head_dim=32, block_size=16, page_size=4, batch=2,
                key_capacity=96, window=2, p_random=0.3, unmapped_frac=unmapped,
                all_blocks=all_blocks, name="tiny_sparse")
    args.update(kw)
    return W.sparse_workload(seed, **args)


def _key_position_rows(sw, b, h):
    """K, V rows [key_capacity, D] of batch b, kv head h in key-position order, plus a mapped
    mask (page id >= 0)."""
    ps, ppb = sw["page_size"], sw["pages_per_block"]
    cap = sw["max_pages"] * ps
    K = np.zeros((cap, sw["D"]))
    V = np.zeros((cap, sw["D"]))
    mapped = np.zeros(cap, dtype=bool)
    for slot in range(sw["max_pages"]):
        pid = sw["block_tables"][b, slot]
        if pid < 0:
            continue
        K[slot * ps:(slot + 1) * ps] = sw["k_pages"][pid, h]
        V[slot * ps:(slot + 1) * ps] = sw["v_pages"][pid, h]
        mapped[slot * ps:(slot + 1) * ps] = True
    del ppb
    return K, V, mapped


def _dense_reference(sw, q_pos=None):
    """For each (q, h) group: SDPA over the keys its edges cover (t < block_len of each edge's
    block) that sit on mapped pages (and, with q_pos, at positions <= q_pos[q]). Returns
    [Tq, hq, D] float64."""
    out = np.zeros((sw["Tq"], sw["hq"], sw["D"]))
    em = sw["edge_meta"]
    gp = sw["group_ptr"]
    bs = sw["block_size"]
    cache = {}
    for q in range(sw["Tq"]):
        for h in range(sw["hkv"]):
            edges = em[gp[q * sw["hkv"] + h]:gp[q * sw["hkv"] + h + 1]]
            if len(edges) == 0:
                continue
            b = int(edges[0, 3])
            if (b, h) not in cache:
                cache[(b, h)] = _key_position_rows(sw, b, h)
            K, V, mapped = cache[(b, h)]
            sel = np.zeros(K.shape[0], dtype=bool)
            for (_, _, blk, _, blen) in edges:
                sel[blk * bs: blk * bs + max(0, blen)] = True
            sel &= mapped
            if q_pos is not None:
                sel &= np.arange(K.shape[0]) <= q_pos[q]
            if not sel.any():
                continue
            qv = torch.from_numpy(sw["q_buf"][q, h * sw["qhead"]:(h + 1) * sw["qhead"]]
                                  .astype(np.float64))[:, None, :]           # [qhead, 1, D]
            k = torch.from_numpy(K[sel])[None].expand(sw["qhead"], -1, -1)
            v = torch.from_numpy(V[sel])[None].expand(sw["qhead"], -1, -1)
            o = F.scaled_dot_product_attention(qv, k, v, scale=sw["softmax_scale"])
            out[q, h * sw["qhead"]:(h + 1) * sw["qhead"]] = o[:, 0].numpy()
    return out


def _merge(oracle, sw, o, m, l):
    return oracle.split_combine(o, m, l, lanes=sw["qhead"], head_dim=sw["D"],
                                group_ptr=sw["group_ptr"], out_dtype=np.float32)


@pytest.mark.parametrize("all_blocks,unmapped", [(True, 0.0), (True, 0.2), (False, 0.0),
                                                 (False, 0.15)])
def test_merged_partials_equal_dense_attention(oracle, all_blocks, unmapped):
    sw = _sw(50, all_blocks=all_blocks, unmapped=unmapped)
    o, m, l = oracle.sparse_forward(sw)
    merged = _merge(oracle, sw, o, m, l).reshape(sw["Tq"], sw["hq"], sw["D"])
    ref = _dense_reference(sw)
    assert np.allclose(merged, ref, rtol=1e-5, atol=1e-6)


def test_zero_length_and_unmapped_blocks_give_sentinel(oracle):
    sw = _sw(51, all_blocks=True)
    em = sw["edge_meta"].copy()
    em[0, 4] = 0           # block_len 0
    em[1, 4] = -3          # negative block_len behaves as 0
    bt = sw["block_tables"].copy()
    b, blk = em[2, 3], em[2, 2]
    ppb = sw["pages_per_block"]
    bt[b, blk * ppb:(blk + 1) * ppb] = -1    # every page of edge 2's block unmapped
    o, m, l = oracle.sparse_forward(sw, edge_meta=em, block_tables=bt)
    for e in (0, 1, 2):
        p = slice(e * sw["qhead"], (e + 1) * sw["qhead"])
        assert np.all(m[p] == np.float32(-1e30))
        assert np.all(l[p] == 0) and np.all(o[p] == 0)


def test_single_key_block_returns_that_value(oracle):
    """block_len = 1: m is that key's score, l = exp(0) = 1, o is its value row exactly."""
    sw = _sw(52, all_blocks=True)
    em = sw["edge_meta"].copy()
    em[:, 4] = 1
    o, m, l = oracle.sparse_forward(sw, edge_meta=em)
    ps = sw["page_size"]
    ppb = sw["pages_per_block"]
    for e in range(0, em.shape[0], 7):
        q_idx, h, blk, b, _ = em[e]
        pid = sw["block_tables"][b, blk * ppb]
        for qh in range(sw["qhead"]):
            p = e * sw["qhead"] + qh
            if pid < 0:
                assert m[p] == np.float32(-1e30) and l[p] == 0
                continue
            assert l[p] == 1.0
            assert np.array_equal(o[p], sw["v_pages"][pid, h, 0])
            s = float(np.dot(sw["q_buf"][q_idx, h * sw["qhead"] + qh].astype(np.float64),
                             sw["k_pages"][pid, h, 0].astype(np.float64))) * sw["softmax_scale"]
            assert m[p] == np.float32(s)
    del ps


def test_partials_are_block_local(oracle):
    """Each partial's m is the max score inside its own block: shifting one block's keys so all
    its scores rise leaves every other edge's partial unchanged."""
    sw = _sw(53, all_blocks=True)
    o, m, l = oracle.sparse_forward(sw)
    sw2 = dict(sw)
    sw2["k_pages"] = sw["k_pages"].copy()
    em = sw["edge_meta"]
    b, blk, h = em[0, 3], em[0, 2], em[0, 1]
    ppb = sw["pages_per_block"]
    for slot in range(blk * ppb, (blk + 1) * ppb):
        pid = sw["block_tables"][b, slot]
        if pid >= 0:
            sw2["k_pages"][pid, h] *= 3.0
    o2, m2, l2 = oracle.sparse_forward(sw2)
    touched = (em[:, 3] == b) & (em[:, 2] == blk) & (em[:, 1] == h)
    rows = np.repeat(~touched, sw["qhead"])
    assert np.array_equal(o[rows], o2[rows]) and np.array_equal(m[rows], m2[rows])
    assert np.array_equal(l[rows], l2[rows])


# ------------------------------------------------------------------ right-aligned causal mask
@pytest.mark.parametrize("all_blocks,unmapped", [(True, 0.0), (True, 0.2), (False, 0.15)])
def test_causal_merged_equals_dense_causal_attention(oracle, all_blocks, unmapped):
    """With q_pos the merged partials equal SDPA over the covered, mapped keys at positions
    <= q_pos[q] (torch, float64)."""
    sw = _sw(60, all_blocks=all_blocks, unmapped=unmapped)
    o, m, l = oracle.sparse_forward(sw, q_pos=sw["q_pos"])
    merged = _merge(oracle, sw, o, m, l).reshape(sw["Tq"], sw["hq"], sw["D"])
    ref = _dense_reference(sw, q_pos=sw["q_pos"])
    assert np.allclose(merged, ref, rtol=1e-5, atol=1e-6)


def test_causal_far_positions_change_nothing(oracle):
    sw = _sw(61, all_blocks=True)
    far = np.full(sw["Tq"], 10 ** 9, dtype=np.int32)
    a = oracle.sparse_forward(sw)
    b = oracle.sparse_forward(sw, q_pos=far)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_causal_blocks_after_the_position_give_sentinel(oracle):
    sw = _sw(62, all_blocks=True)
    em = sw["edge_meta"]
    o, m, l = oracle.sparse_forward(sw, q_pos=sw["q_pos"])
    after = em[:, 2] * sw["block_size"] > sw["q_pos"][em[:, 0]]
    assert after.any()
    rows = np.repeat(after, sw["qhead"])
    assert np.all(o[rows] == 0) and np.all(m[rows] == np.float32(-1e30)) and np.all(l[rows] == 0)


def test_causal_equals_block_cut_at_the_position(oracle):
    """An edge whose block holds the query position gives the same bits as the unmasked edge with
    block_len cut to q_pos - blk * block_size + 1: the mask is a prefix of the block."""
    sw = _sw(63, all_blocks=True)
    em = sw["edge_meta"].copy()
    qp = sw["q_pos"][em[:, 0]]
    start = em[:, 2] * sw["block_size"]
    inside = (qp >= start) & (qp - start + 1 < em[:, 4])
    assert inside.any()
    cut = em.copy()
    cut[inside, 4] = (qp - start + 1)[inside]
    a = oracle.sparse_forward(sw, q_pos=sw["q_pos"])
    b = oracle.sparse_forward(sw, edge_meta=cut)
    rows = np.repeat(inside, sw["qhead"])
    for x, y in zip(a, b):
        assert np.array_equal(x[rows], y[rows])


# ------------------------------------------------------------------ edge-list builder
@pytest.mark.parametrize("all_blocks", [False, True])
def test_built_edges_equal_the_generators(oracle, all_blocks):
    """The generator forms its edges with numpy (nonzero of the mask in row-major order, block_len
    clipped by numpy); the oracle's loop gives the same list and CSR offsets."""
    sw = _sw(70, all_blocks=all_blocks, Tq=20, key_capacity=160)
    em, gp = oracle.build_edges(sw["block_mask"], sw["q_batch"], sw["used_kv_lens"],
                                sw["block_size"])
    assert np.array_equal(em, sw["edge_meta"])
    assert np.array_equal(gp, sw["group_ptr"])


def test_built_edges_counts_and_lengths(oracle):
    rng = np.random.default_rng(71)
    tq, hkv, nblk, bs = 7, 3, 11, 16
    mask = (rng.random((tq, hkv, nblk)) < 0.4).astype(np.uint8)
    mask[2] = 0                                    # a row with no edge at all
    q_batch = rng.integers(0, 2, size=tq).astype(np.int32)
    used = np.array([5 * bs + 3, 0], dtype=np.int32)   # batch 1 has no keys
    em, gp = oracle.build_edges(mask, q_batch, used, bs)
    assert np.array_equal(np.diff(gp), mask.reshape(tq * hkv, nblk).sum(axis=1))
    assert gp[-1] == len(em) == int(mask.sum())
    blk, b, blen = em[:, 2], em[:, 3], em[:, 4]
    assert np.array_equal(b, q_batch[em[:, 0]])
    assert np.all(blen[b == 1] == 0)
    full = (b == 0) & (blk < 5)
    assert np.all(blen[full] == bs) and np.all(blen[(b == 0) & (blk == 5)] == 3)
    assert np.all(blen[(b == 0) & (blk > 5)] == 0)
    # sorted by (q, h, blk)
    key = (em[:, 0].astype(np.int64) * hkv + em[:, 1]) * nblk + blk
    assert np.all(np.diff(key) > 0)


def test_built_edges_empty_mask(oracle):
    em, gp = oracle.build_edges(np.zeros((4, 2, 5), np.uint8), np.zeros(4, np.int32),
                                np.array([70], np.int32), 16)
    assert len(em) == 0 and np.all(gp == 0)
