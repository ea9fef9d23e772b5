"""Pins of the oracle's paged attention, split partials and log-sum-exp merge.

Pages: PagedAttention manifest (inputs, is_causal, qPerKv head grouping, split-K passes, merge),
and the block-sparse forward page (natural-log online softmax, (o, m, l) partials).
The library pin is torch's scaled_dot_product_attention in float64 on the CPU; the paged path
with a contiguous block table must reduce to it.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from block_sparse_gqa_paged_amd import workloads as W


def _wl(seed, past, n_new, H=4, G=2, D=64, bs=16, table="pool", packed=False, causal=1, **kw):
    return W.paged_workload(seed, past=past, n_new=n_new, num_heads=H, kv_num_heads=G,
                            head_size=D, block_size=bs, table=table, slack=0.3, packed=packed,
                            causal=causal, name="t", **kw)


def _dense_kv(w):
    """Per-sequence contiguous K, V [L_b, G, D] read through the block table (float64)."""
    out = []
    for b in range(w["B"]):
        L = int(w["past"][b] + w["cu"][b + 1] - w["cu"][b])
        blocks = w["block_table"][b, :(L + w["bs"] - 1) // w["bs"]]
        k = w["key_cache"][blocks].reshape(-1, w["G"], w["D"])[:L].astype(np.float64)
        v = w["value_cache"][blocks].reshape(-1, w["G"], w["D"])[:L].astype(np.float64)
        out.append((k, v))
    return out


def _sdpa_reference(w, causal=None):
    """torch SDPA in float64: each sequence's new rows attend to its keys, kv heads repeated
    qPerKv times (head h uses kv head h // qPerKv), with a causal mask that offsets queries by
    past_b when causal."""
    causal = w["causal"] if causal is None else causal
    H, G, D = w["H"], w["G"], w["D"]
    Q = H // G
    qs = (H + 2 * G) * D if w["packed"] else H * D
    q_all = w["query"].reshape(w["T"], qs)[:, :H * D].astype(np.float64).reshape(w["T"], H, D)
    out = np.zeros((w["T"], H, D))
    for b, (k, v) in enumerate(_dense_kv(w)):
        r0, r1 = w["cu"][b], w["cu"][b + 1]
        n = r1 - r0
        if n == 0:
            continue
        L = k.shape[0]
        q = torch.from_numpy(q_all[r0:r1]).permute(1, 0, 2)                   # [H, n, D]
        kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(Q, dim=0)  # [H, L, D]
        vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(Q, dim=0)
        if causal:
            qpos = w["past"][b] + torch.arange(n)
            mask = torch.arange(L)[None, :] <= qpos[:, None]
        else:
            mask = torch.ones(n, L, dtype=torch.bool)
        o = F.scaled_dot_product_attention(q, kt, vt, attn_mask=mask, scale=w["scale"])
        out[r0:r1] = o.permute(1, 0, 2).numpy()
    return out.reshape(w["T"], H * D)


def _assert_fp16_close(got, ref_f64, ulps=1):
    """got (fp16) is the fp16 rounding of ref within `ulps` fp16 ulps."""
    g = got.astype(np.float64)
    sp = np.spacing(np.abs(ref_f64).astype(np.float16)).astype(np.float64)
    err = np.abs(g - ref_f64)
    assert np.all(err <= ulps * sp + 1e-7), float((err / (sp + 1e-30)).max())


CASES = [
    dict(seed=20, past=[37, 100], n_new=[1, 1]),                          # decode, Q=2
    dict(seed=21, past=[0, 5, 60], n_new=[7, 1, 20], bs=8),               # prefill + decode
    dict(seed=22, past=[3, 0], n_new=[40, 33], H=8, G=2, D=128, bs=32),   # Q=4, D=128
    dict(seed=23, past=[17], n_new=[5], H=3, G=3, D=64, bs=1),            # Q=1, block size 1
    dict(seed=24, past=[9, 12], n_new=[4, 2], H=8, G=1, bs=16, packed=True),  # MQA, packed
    dict(seed=25, past=[0, 0, 4], n_new=[1, 0, 3], bs=4),                 # empty sequence
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: str(c["seed"]))
@pytest.mark.parametrize("causal", [1, 0])
def test_dense_matches_sdpa(oracle, case, causal):
    case = dict(case)
    w = _wl(case.pop("seed"), causal=causal, **case)
    got = oracle.paged_attention(w)
    _assert_fp16_close(got, _sdpa_reference(w))


def test_single_visible_key_returns_value_exactly(oracle):
    """past = 0, one new token, causal: the only visible key gets weight exp(0)/1 = 1."""
    w = _wl(30, past=[0, 0], n_new=[1, 1], H=4, G=2)
    out = oracle.paged_attention(w)
    for b in range(2):
        blk = w["block_table"][b, 0]
        v = w["value_cache"][blk, 0]                    # [G, D]
        expect = np.repeat(v, 2, axis=0).reshape(-1)    # heads 2g, 2g+1 use kv head g
        assert np.array_equal(out[b].view(np.uint16), expect.view(np.uint16))


def test_uniform_scores_give_mean_of_values(oracle):
    """q = 0 makes every score 0, so the output is the plain mean of the visible values."""
    w = _wl(31, past=[50, 7], n_new=[1, 1], H=4, G=2)
    w["query"] = np.zeros_like(w["query"])
    out = oracle.paged_attention(w).reshape(2, 4, -1)
    for b, (k, v) in enumerate(_dense_kv(w)):
        mean = v.mean(axis=0)                           # [G, D]
        _assert_fp16_close(out[b], np.repeat(mean, 2, axis=0))


def test_page_permutation_is_bit_identical(oracle):
    w = _wl(32, past=[70, 3, 33], n_new=[1, 9, 2], bs=8)
    a = oracle.paged_attention(w)
    perm = np.random.default_rng(1).permutation(w["NB"])
    inv = np.argsort(perm)
    w2 = dict(w)
    w2["key_cache"], w2["value_cache"] = w["key_cache"][perm], w["value_cache"][perm]
    bt = w["block_table"].copy()
    bt[bt >= 0] = inv[bt[bt >= 0]]
    w2["block_table"] = bt
    b = oracle.paged_attention(w2)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_stale_nan_rows_are_never_read(oracle):
    """NaN in every cache row beyond each sequence's length must not reach the output."""
    w = _wl(33, past=[20, 45], n_new=[3, 1], poison=True)
    out = oracle.paged_attention(w)
    assert np.isfinite(out.astype(np.float32)).all()
    _assert_fp16_close(out, _sdpa_reference(w))


# ------------------------------------------------------------------ split partials + merge
@pytest.mark.parametrize("S", [1, 2, 3, 7, 16])
def test_split_merge_matches_dense(oracle, S):
    w = _wl(40, past=[100, 0, 250], n_new=[1, 5, 1], bs=16)
    o, m, l = oracle.paged_attention_partials(w, S)
    merged = oracle.split_combine(o, m, l, lanes=w["H"], head_dim=w["D"], num_splits=S,
                                  out_dtype=np.float32)
    ref = _sdpa_reference(w)
    assert np.allclose(merged.reshape(ref.shape), ref, rtol=1e-6, atol=1e-6)


def test_single_split_is_o_over_l(oracle):
    w = _wl(41, past=[30, 64], n_new=[1, 1])
    o, m, l = oracle.paged_attention_partials(w, 1)
    dense = oracle.paged_attention(w).reshape(-1, w["D"])
    assert np.array_equal((o / l[:, None]).astype(np.float16).view(np.uint16),
                          dense.view(np.uint16))


def test_fixed_chunk_partials_and_empty_sentinel(oracle):
    """chunk_keys fixes the chunk; chunks past the visible keys emit (0, -1e30, 0)."""
    w = _wl(42, past=[40], n_new=[1], H=2, G=1)
    o, m, l = oracle.paged_attention_partials(w, 4, chunk_keys=16)   # 41 keys: 16+16+9+empty
    last = np.arange(3, 4 * 2, 4)                                   # split 3 of both heads
    assert np.all(m.reshape(4, 2)[3] == np.float32(-1e30))
    assert np.all(l.reshape(4, 2)[3] == 0) and np.all(o.reshape(4, 2, -1)[3] == 0)
    assert last.size == 2
    merged = oracle.split_combine(o, m, l, lanes=2, head_dim=w["D"], num_splits=4,
                                  out_dtype=np.float32)
    assert np.allclose(merged.reshape(1, -1), _sdpa_reference(w), rtol=1e-6, atol=1e-6)


def test_combine_closed_form(oracle):
    """Two partials with l = 1 and 3 at the same max weigh their sums 1:1; shifting one max by
    ln 2 doubles its weight; an l = 0 sentinel is ignored."""
    D = 4
    o = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [9e9, 9e9, 9e9, 9e9]], np.float32)
    m = np.array([0.5, 0.5, -1e30], np.float32)
    l = np.array([1.0, 3.0, 0.0], np.float32)
    out = oracle.split_combine(o, m, l, lanes=1, head_dim=D, group_ptr=np.array([0, 3]),
                               out_dtype=np.float32)
    assert np.allclose(out[0], (o[0] + o[1]) / 4.0, rtol=1e-7)
    m2 = np.array([0.0, np.log(2.0), -1e30], np.float32)
    out2 = oracle.split_combine(o, m2, l, lanes=1, head_dim=D, group_ptr=np.array([0, 3]),
                                out_dtype=np.float32)
    w1 = np.exp(np.float64(m2[0]) - np.float64(m2[1]))
    assert np.allclose(out2[0], (w1 * o[0] + o[1]) / (w1 * 1 + 3), rtol=1e-6)
    # an empty group and an all-sentinel group both give 0
    out3 = oracle.split_combine(o, m, l, lanes=1, head_dim=D, group_ptr=np.array([0, 0, 0, 3]),
                                out_dtype=np.float32)
    assert np.all(out3[:2] == 0)
    out4 = oracle.split_combine(o[2:], m[2:], l[2:], lanes=1, head_dim=D,
                                group_ptr=np.array([0, 1]), out_dtype=np.float32)
    assert np.all(out4 == 0)


def test_combine_is_order_invariant(oracle):
    w = _wl(43, past=[300, 77], n_new=[1, 1], bs=16)
    S = 5
    o, m, l = oracle.paged_attention_partials(w, S)
    H = w["H"]
    a = oracle.split_combine(o, m, l, lanes=H, head_dim=w["D"], num_splits=S,
                             out_dtype=np.float32)
    # reverse the splits of every token via a CSR layout over permuted partial units
    order = np.concatenate([np.arange(S)[::-1] + t * S for t in range(w["T"])])
    o2 = o.reshape(-1, H, w["D"])[order].reshape(o.shape)
    m2 = m.reshape(-1, H)[order].reshape(-1)
    l2 = l.reshape(-1, H)[order].reshape(-1)
    gp = np.arange(0, w["T"] * S + 1, S)
    b = oracle.split_combine(o2, m2, l2, lanes=H, head_dim=w["D"], group_ptr=gp,
                             out_dtype=np.float32)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-7)
