"""GPU parity of the block-sparse edge forward (pa_sparse_forward) and its merge against the CPU
oracle: tiny edge lists compared partial by partial, inputs with a wide dynamic range (outlier
channels, rows near 1e-5), and the full-size workload (Tq 4096, hkv 8, qhead 4, D 128, block 64,
page 16) compared on every merged row and on every partial of a seeded 1% edge sample.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_gqa_paged_amd as pa  # noqa: E402
import oracle  # noqa: E402
from block_sparse_gqa_paged_amd import device as dev  # noqa: E402
from block_sparse_gqa_paged_amd import workloads as W  # noqa: E402
from parity import (assert_bits_equal, assert_sparse_out_close,  # noqa: E402
                    assert_sparse_partials_close, oracle_sparse_full)

pytestmark = pytest.mark.gpu


def _tiny(seed, **kw):
    args = dict(Tq=24, hkv=2, qhead=4, head_dim=128, block_size=64, page_size=16, batch=2,
                key_capacity=512, window=2, p_random=0.3, unmapped_frac=0.15, name="tiny")
    args.update(kw)
    return W.sparse_workload(seed, **args)


TINY = [
    dict(seed=200),
    dict(seed=201, head_dim=64, block_size=32, page_size=8, qhead=2),
    dict(seed=202, qhead=1, hkv=3, block_size=16, page_size=16, unmapped_frac=0.0),
    dict(seed=203, qhead=8, block_size=128, page_size=32, head_dim=64, key_capacity=1024),
    dict(seed=204, qhead=3, block_size=48, page_size=16, key_capacity=480, all_blocks=True),
    # 128-key blocks at D = 128: the largest LDS footprint
    dict(seed=205, block_size=128, page_size=16, key_capacity=1024),
    # many edges per key block: several work items share one block
    dict(seed=206, Tq=600, hkv=1, qhead=2, key_capacity=256, window=3, p_random=0.5),
    # one edge per 16-row group
    dict(seed=207, qhead=16, hkv=1, head_dim=64, block_size=32, page_size=8),
    # head dim 256 (blocks of up to 64 keys)
    dict(seed=208, head_dim=256, block_size=64, page_size=16),
    dict(seed=209, head_dim=256, block_size=32, page_size=8, qhead=2),
    # q-head lanes beyond one 16-row group: an edge's rows span groups
    dict(seed=212, qhead=32, hkv=1, head_dim=64, block_size=32, page_size=8),
    dict(seed=213, qhead=24, hkv=2, head_dim=128),
    # more key blocks (17002) than the LDS histogram of the chunked edge sort holds: the sort
    # takes its global-atomic form
    dict(seed=216, hkv=1, qhead=2, head_dim=64, block_size=16, page_size=16,
         key_capacity=16 * 8500, p_random=0.02),
]


@pytest.mark.parametrize("case", TINY, ids=lambda c: str(c["seed"]))
def test_tiny_partials_and_merge(case):
    case = dict(case)
    sw = _tiny(case.pop("seed"), **case)
    ref = oracle.sparse_forward(sw)
    c = dev.SparseCase(sw)
    got = c.forward()
    out = c.combine()
    torch.cuda.synchronize()
    assert_sparse_partials_close(got, ref, "partials")
    merged = oracle.split_combine(*ref, lanes=sw["qhead"], head_dim=sw["D"],
                                  group_ptr=sw["group_ptr"], out_dtype=np.float32)
    assert_sparse_out_close(out, merged, "merged")


@pytest.mark.parametrize("case", TINY[:4] + TINY[5:], ids=lambda c: str(c["seed"]))
def test_tiny_causal_partials_and_merge(case):
    """Right-aligned causal mask: partials and merged rows against the oracle with q_pos."""
    case = dict(case)
    sw = _tiny(case.pop("seed"), **case)
    ref = oracle.sparse_forward(sw, q_pos=sw["q_pos"])
    c = dev.SparseCase(sw)
    got = c.forward(causal=True)
    out = c.combine()
    torch.cuda.synchronize()
    assert_sparse_partials_close(got, ref, "causal partials")
    merged = oracle.split_combine(*ref, lanes=sw["qhead"], head_dim=sw["D"],
                                  group_ptr=sw["group_ptr"], out_dtype=np.float32)
    assert_sparse_out_close(out, merged, "causal merged")


# Wide dynamic range inside key blocks, value dimensions and query rows: outlier channels (keys
# and values x100 / x1000, the matching query channels scaled down so scores stay O(1)) and rows
# near 1e-5, at the 1e-4 bar. In an outlier value channel the weighted sum of terms of size ~1000
# can cancel to a small value; its fp32 rounding is relative to the terms (the page's own loops
# run in plain fp32 miss 1e-4 * max(1, |o|) by up to 6x there, and stay near 1e-6 of the terms),
# so o and the merged rows are held to 1e-4 of the magnitude of their terms.
WIDE = [
    dict(seed=220, outliers=(3, 1000.0, 1000.0)),
    dict(seed=221, outliers=(3, 100.0, 100.0), tiny=(0.1, 1e-5)),
    dict(seed=222, tiny=(0.25, 1e-5)),
    dict(seed=223, head_dim=64, block_size=32, page_size=8, qhead=2,
         outliers=(2, 1000.0, 100.0), tiny=(0.1, 1e-5)),
    dict(seed=224, qhead=8, block_size=128, page_size=32, outliers=(4, 300.0, 1000.0),
         tiny=(0.05, 1e-5), key_capacity=1024),
    dict(seed=225, head_dim=256, outliers=(3, 1000.0, 1000.0), tiny=(0.1, 1e-5)),
]


def _assert_wide(sw):
    """The inputs really span the range: within key rows (outliers) and between rows (tiny)."""
    k = np.abs(sw["k_pages"]).reshape(-1, sw["D"])
    v = np.abs(sw["v_pages"]).reshape(-1, sw["D"])
    spread = [np.median(x.max(axis=1) / np.maximum(np.median(x, axis=1), 1e-30)) for x in (k, v)]
    tiny = [(x.max(axis=1) < 1e-3 * np.median(x.max(axis=1))).mean() for x in (k, v)]
    return spread, tiny


@pytest.mark.parametrize("case", WIDE, ids=lambda c: str(c["seed"]))
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_wide_dynamic_range(case, causal):
    case = dict(case)
    sw = _tiny(case.pop("seed"), **case)
    spread, tiny = _assert_wide(sw)
    if "outliers" in case:
        assert min(spread) > 50, spread        # each row's max far above its typical element
    if "tiny" in case:
        assert min(tiny) > 0.02, tiny          # rows near 1e-5 inside the blocks
    q_pos = sw["q_pos"] if causal else None
    ref = oracle.sparse_forward(sw, q_pos=q_pos)
    # the magnitude of the summed terms: the same partials over |V| (the weights do not change)
    o_terms = oracle.sparse_forward(dict(sw, v_pages=np.abs(sw["v_pages"])), q_pos=q_pos)[0]
    c = dev.SparseCase(sw)
    got = c.forward(causal=causal)
    out = c.combine()
    torch.cuda.synchronize()
    assert_sparse_partials_close(got, ref, "wide partials", o_terms=o_terms)
    kw = dict(lanes=sw["qhead"], head_dim=sw["D"], group_ptr=sw["group_ptr"],
              out_dtype=np.float32)
    merged = oracle.split_combine(*ref, **kw)
    terms = oracle.split_combine(o_terms, ref[1], ref[2], **kw)
    assert_sparse_out_close(out, merged, "wide merged", terms=terms)


def _poison_past_used(sw):
    """Copy of sw whose cache rows at key positions >= each batch's used length (on mapped
    pages) hold NaN: rows that no edge reads (block_len stops before them)."""
    k, v = sw["k_pages"].copy(), sw["v_pages"].copy()
    ps, n = sw["page_size"], 0
    for b in range(sw["batch"]):
        used = int(sw["used_kv_lens"][b])
        for t in range(used, sw["max_pages"] * ps):
            pid = int(sw["block_tables"][b, t // ps])
            if pid < 0:
                continue
            k[pid, :, t % ps, :] = np.nan
            v[pid, :, t % ps, :] = np.nan
            n += 1
    assert n > 0
    return dict(sw, k_pages=k, v_pages=v)


@pytest.mark.parametrize("seed,kw", [(214, {}), (215, dict(head_dim=64, block_size=32,
                                                            page_size=8, qhead=2))],
                         ids=["d128", "d64"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_poison_past_used_length(seed, kw, causal):
    """Rows past the used length do not reach the partials: the result equals the oracle's on
    the clean cache (the oracle never reads those rows, so its result is the same either way)."""
    sw = _tiny(seed, **kw)
    q_pos = sw["q_pos"] if causal else None
    ref = oracle.sparse_forward(sw, q_pos=q_pos)
    bad = _poison_past_used(sw)
    ref_bad = oracle.sparse_forward(bad, q_pos=q_pos)
    for x, y in zip(ref, ref_bad):
        np.testing.assert_array_equal(x, y)
    c = dev.SparseCase(bad)
    got = c.forward(causal=causal)
    torch.cuda.synchronize()
    for t in got:
        assert torch.isfinite(t).all()
    assert_sparse_partials_close(got, ref, "poisoned partials")


def test_magnitudes_far_below_one():
    """Query rows and key blocks near 1e-36 and values near 1e-39 (fp32 subnormals): the power
    of two that scales each row, block or value dimension up before the fp16 split is capped so
    that it stays finite. Scores underflow to 0 on both sides (uniform weights); the partials
    stay finite and o matches the oracle's relative to its largest element."""
    sw = _tiny(217, head_dim=64, block_size=32, page_size=8, qhead=2)
    sw = dict(sw, q_buf=sw["q_buf"] * np.float32(1e-36), k_pages=sw["k_pages"] * np.float32(1e-36),
              v_pages=sw["v_pages"] * np.float32(1e-39))
    ref = oracle.sparse_forward(sw)
    c = dev.SparseCase(sw)
    o, m, l = (t.cpu().numpy() for t in c.forward())
    for t in (o, m, l):
        assert np.isfinite(t).all()
    np.testing.assert_allclose(m, ref[1], atol=1e-4)
    np.testing.assert_allclose(l, ref[2], rtol=1e-5, atol=1e-5)
    scale = np.abs(ref[0]).max()
    assert scale > 0
    assert np.abs(o - ref[0]).max() <= 1e-3 * scale, np.abs(o - ref[0]).max() / scale


def test_sentinels_and_out_of_range_edges():
    sw = _tiny(210)
    em = sw["edge_meta"].copy()
    em[0, 4] = 0                       # empty block
    em[1, 4] = -5
    bt = sw["block_tables"].copy()
    b, blk = em[2, 3], em[2, 2]
    bt[b, blk * 4:(blk + 1) * 4] = -1  # every page of edge 2's block unmapped
    sw = dict(sw, edge_meta=em, block_tables=bt)
    ref = oracle.sparse_forward(sw)
    c = dev.SparseCase(sw)
    o, m, l = c.forward()
    torch.cuda.synchronize()
    assert_sparse_partials_close((o, m, l), ref)
    for e in (0, 1, 2):
        p = slice(4 * e, 4 * e + 4)
        assert np.all(m[p].cpu().numpy() == np.float32(-1e30))
        assert np.all(l[p].cpu().numpy() == 0) and np.all(o[p].cpu().numpy() == 0)


def test_edge_order_does_not_change_results():
    sw = _tiny(211)
    c = dev.SparseCase(sw)
    a = [x.cpu().numpy().copy() for x in c.forward()]
    perm = np.random.default_rng(2).permutation(sw["E"])
    sw2 = dict(sw, edge_meta=sw["edge_meta"][perm])
    c2 = dev.SparseCase(sw2)
    b = [x.cpu().numpy() for x in c2.forward()]
    q = sw["qhead"]
    rows = (perm[:, None] * q + np.arange(q)[None, :]).reshape(-1)
    for x, y in zip(a, b):
        assert np.array_equal(x[rows], y)


@pytest.fixture(scope="module")
def full():
    sw = W.block_sparse_forward()
    c = dev.SparseCase(sw)
    o, m, l = c.forward()
    out = c.combine()
    torch.cuda.synchronize()
    return sw, o.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy(), out.cpu().numpy()


def _check_full(sw, o, m, l, out, q_pos=None):
    """Every merged row against the oracle's, and every partial of a seeded 1% edge sample."""
    rng = np.random.default_rng(7)
    sample = np.sort(rng.choice(sw["E"], size=max(1, sw["E"] // 100), replace=False))
    merged, (ro, rm, rl) = oracle_sparse_full(oracle, sw, q_pos=q_pos, sample_edges=sample)
    q = sw["qhead"]
    prow = (sample[:, None] * q + np.arange(q)[None, :]).reshape(-1)
    assert_sparse_partials_close((o[prow], m[prow], l[prow]), (ro, rm, rl), "1% edge sample")
    assert_sparse_out_close(out, merged, "every merged row")


def test_full_size_every_merged_row(full):
    _check_full(*full)


def test_full_size_causal_every_merged_row(full):
    """The same workload under the right-aligned causal mask (its random blocks past a row's
    position become sentinels, the row's own block is cut at the position)."""
    sw = full[0]
    c = dev.SparseCase(sw)
    o, m, l = c.forward(causal=True)
    out = c.combine()
    torch.cuda.synchronize()
    _check_full(sw, o.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy(), out.cpu().numpy(),
                q_pos=sw["q_pos"])


def test_full_size_invariants(full):
    sw, o, m, l, out = full
    assert np.isfinite(out).all() and np.isfinite(o).all()
    # every mapped edge has l >= 1 (its max key contributes exp(0)); unmapped blocks l == 0
    assert (l >= 0).all()
    pos = l > 0
    assert (l[pos] >= 1.0 - 1e-6).all()
    assert np.all(m[~pos] == np.float32(-1e30))


# The forward (its edge sort and its main kernel) and the merge captured into one HIP graph. The
# library enqueues kernels only (the sort's counters and histograms are cleared by its own
# kernels, no memset): every replay, with eager library work between replays, is bit-identical
# to the eager calls. Two sorts: the chunked one (several work items per key block) and the
# global-atomic one (17002 key blocks).
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("kw", [
    dict(seed=217, Tq=600, hkv=1, qhead=2, key_capacity=256, window=3, p_random=0.5),
    dict(seed=218, hkv=1, qhead=2, head_dim=64, block_size=16, page_size=16,
         key_capacity=16 * 8500, p_random=0.02),
], ids=["chunked_sort", "global_sort"])
def test_graph_capture_replays_match_eager(kw, causal):
    kw = dict(kw)
    sw = _tiny(kw.pop("seed"), **kw)
    c = dev.SparseCase(sw)

    def step():
        c.forward(causal=causal)
        c.combine()

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (c.o, c.m, c.l, c.out)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    names = ("o", "m", "l", "merged")
    for i in range(3):
        for x in (c.o, c.m, c.l, c.out):
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, r, n in zip((c.o, c.m, c.l, c.out), ref, names):
            assert_bits_equal(x, r, f"{n} after replay {i}")
        step()
        torch.cuda.synchronize()
        for x, r, n in zip((c.o, c.m, c.l, c.out), ref, names):
            assert_bits_equal(x, r, f"eager {n} after replay {i}")
