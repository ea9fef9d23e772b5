"""GPU parity of the block-sparse edge-list builder (pa_sparse_build_edges) against the oracle:
every edge and CSR offset bit for bit, on random masks (empty rows, nblk below, at and above 64
and not a multiple of it, rows of batches with few or no keys), on the full block-sparse
workload's mask (whose edges the generator also forms on the host), and with a capacity smaller
than the edge count.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from block_sparse_gqa_paged_amd import device as dev  # noqa: E402
from block_sparse_gqa_paged_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu


def _random_case(seed, tq, hkv, nblk, batch, density, block_size=16):
    rng = np.random.default_rng(seed)
    mask = (rng.random((tq, hkv, nblk)) < density).astype(np.uint8)
    if tq > 2:
        mask[1] = 0                                   # a query row with no edge at all
    q_batch = rng.integers(0, batch, size=tq).astype(np.int32)
    used = rng.integers(0, nblk * block_size + 1, size=batch).astype(np.int32)
    used[0] = 0                                       # a batch with no keys: every len is 0
    return dict(block_mask=mask, q_batch=q_batch, used_kv_lens=used, block_size=block_size,
                batch=batch)


CASES = [
    dict(seed=300, tq=5, hkv=3, nblk=11, batch=2, density=0.5),
    dict(seed=301, tq=9, hkv=2, nblk=64, batch=3, density=0.3),
    dict(seed=302, tq=33, hkv=4, nblk=130, batch=2, density=0.1),
    dict(seed=303, tq=70, hkv=1, nblk=1, batch=4, density=0.7),
    dict(seed=304, tq=3, hkv=8, nblk=512, batch=1, density=0.9),
    # 16-byte path: nblk = 16 * 2^k up to 1024, row counts that leave partial loads
    dict(seed=306, tq=37, hkv=3, nblk=16, batch=2, density=0.5),
    dict(seed=307, tq=11, hkv=5, nblk=128, batch=3, density=0.2),
    dict(seed=308, tq=9, hkv=2, nblk=1024, batch=2, density=0.05),
    dict(seed=309, tq=200, hkv=8, nblk=512, batch=2, density=0.06),
    dict(seed=311, tq=45, hkv=3, nblk=256, batch=2, density=0.1),    # 4 rows per load
    dict(seed=312, tq=300, hkv=8, nblk=64, batch=3, density=0.08),   # many workgroups
    # denser rows at the workload's nblk: about 490 and 320 edges per 8 rows
    dict(seed=313, tq=64, hkv=8, nblk=512, batch=2, density=0.12),
    dict(seed=314, tq=64, hkv=8, nblk=512, batch=2, density=0.078),
    # 16 blocks per row, 32 rows per workgroup: 4096 workgroups (each emit workgroup sums the
    # totals before it) and 4100 (the separate offset scan)
    dict(seed=315, tq=16384, hkv=8, nblk=16, batch=3, density=0.3),
    dict(seed=316, tq=16400, hkv=8, nblk=16, batch=3, density=0.3),
]


def _check(sw, capacity=None):
    em_ref, gp_ref = oracle.build_edges(sw["block_mask"], sw["q_batch"], sw["used_kv_lens"],
                                        sw["block_size"])
    b = dev.EdgeBuilder(sw, capacity=capacity)
    em, gp = b.build()
    torch.cuda.synchronize()
    gp = gp.cpu().numpy()
    assert np.array_equal(gp, gp_ref), "group_ptr"
    E = int(gp[-1])
    n = E if capacity is None else min(E, capacity)
    assert np.array_equal(em.cpu().numpy()[:n], em_ref[:n]), "edge_meta"


@pytest.mark.parametrize("case", CASES, ids=lambda c: str(c["seed"]))
def test_random_masks(case):
    _check(_random_case(**case))


def test_empty_query_set():
    _check(dict(block_mask=np.zeros((0, 2, 8), np.uint8), q_batch=np.zeros(0, np.int32),
                used_kv_lens=np.array([5], np.int32), block_size=16, batch=1))


@pytest.mark.parametrize("nblk", [40, 64])
def test_capacity_below_edge_count(nblk):
    sw = _random_case(305, tq=20, hkv=2, nblk=nblk, batch=2, density=0.5)
    _check(sw, capacity=int(sw["block_mask"].sum()) // 3)


def test_nonbinary_mask_bytes():
    """Any nonzero byte keeps its block (on both paths)."""
    for nblk in (24, 32):
        sw = _random_case(310, tq=6, hkv=2, nblk=nblk, batch=2, density=0.5)
        rng = np.random.default_rng(311)
        sw["block_mask"] = (sw["block_mask"] * rng.integers(1, 256, size=sw["block_mask"].shape)
                            ).astype(np.uint8)
        _check(sw)


def test_full_block_sparse_mask():
    """The 0.99 M-edge workload: the device list equals the generator's own host-built list."""
    sw = W.block_sparse_forward()
    b = dev.EdgeBuilder(sw)
    em, gp = b.build()
    torch.cuda.synchronize()
    gp = gp.cpu().numpy()
    assert np.array_equal(gp, sw["group_ptr"])
    assert np.array_equal(em.cpu().numpy()[:sw["E"]], sw["edge_meta"])


@pytest.mark.parametrize("nblk", [64, 40], ids=["16_byte_path", "row_path"])
def test_graph_capture_replays_match_eager(nblk):
    """The edge builder captured into a HIP graph: every replay rewrites the same edges and
    offsets, bit for bit."""
    sw = _random_case(317, tq=300, hkv=8, nblk=nblk, batch=3, density=0.08)
    b = dev.EdgeBuilder(sw)
    em, gp = b.build()
    torch.cuda.synchronize()
    E = int(gp[-1].item())
    ref_em, ref_gp = em[:E].clone(), gp.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.build()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.build()
    for i in range(3):
        em.fill_(-1)
        gp.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(em[:E], ref_em), f"edge_meta after replay {i}"
        assert torch.equal(gp, ref_gp), f"group_ptr after replay {i}"
