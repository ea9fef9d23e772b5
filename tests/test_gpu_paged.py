"""GPU parity of the paged path (pa_kv_append, pa_paged_attention, pa_split_combine) against
the CPU oracle, on seeded workloads: a tiny family that spans several 32-key tiles with ragged
tails, the four paged workload shapes at full size (every output row), NaN in stale cache rows,
page permutation, every split policy, and prefill columns whose running maximum is raised.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_gqa_paged_amd as pa  # noqa: E402
import oracle  # noqa: E402
from block_sparse_gqa_paged_amd import device as dev  # noqa: E402
from block_sparse_gqa_paged_amd import workloads as W  # noqa: E402
from parity import (assert_attention_close, assert_bits_equal, oracle_rows,  # noqa: E402
                    ROT_ABS)
from lazy_softmax import RAISE_CASES, raise_columns  # noqa: E402

pytestmark = pytest.mark.gpu

SPLITS = [pa.PA_SPLITS_AUTO, pa.PA_SPLITS_PAGE_RULE, 1, 2, 3, 16]


def _run(w, num_splits=pa.PA_SPLITS_AUTO, use_slot_mapping=True):
    c = dev.PagedCase(w)
    c.append(use_slot_mapping=use_slot_mapping)
    out = c.attention(num_splits)
    torch.cuda.synchronize()
    return c, out


def _oracle(w):
    kc, vc = oracle.kv_append(w)
    return kc, vc, oracle.paged_attention(w, kc, vc)


TINY = [
    dict(seed=100, past=[37, 100], n_new=[1, 1], num_heads=4, kv_num_heads=2, head_size=64,
         block_size=16),
    dict(seed=101, past=[0, 5, 290, 64], n_new=[9, 1, 1, 40], num_heads=8, kv_num_heads=2,
         head_size=128, block_size=16),
    dict(seed=102, past=[31, 33], n_new=[2, 3], num_heads=4, kv_num_heads=4, head_size=128,
         block_size=32),                                              # Q = 1, 2-3 token decode
    dict(seed=103, past=[17, 3], n_new=[5, 70], num_heads=6, kv_num_heads=2, head_size=64,
         block_size=5),                                               # bs not a power of two
    dict(seed=104, past=[200, 0, 7], n_new=[1, 0, 2], num_heads=16, kv_num_heads=1,
         head_size=64, block_size=8),                                 # MQA, empty sequence
    dict(seed=105, past=[100, 12], n_new=[3, 19], num_heads=8, kv_num_heads=8, head_size=128,
         block_size=64, packed=True, rotary_mode=W.ROTARY_NEOX, rotary_dim=128,
         rotary_positions=256),
    dict(seed=106, past=[45], n_new=[2], num_heads=32, kv_num_heads=1, head_size=64,
         block_size=16, rotary_mode=W.ROTARY_INTERLEAVED, rotary_dim=32, rotary_positions=64),
    dict(seed=107, past=[130, 257], n_new=[1, 1], num_heads=64, kv_num_heads=2, head_size=128,
         block_size=16),                                              # qPerKv 32: two blocks
]


@pytest.mark.parametrize("case", TINY, ids=lambda c: str(c["seed"]))
@pytest.mark.parametrize("num_splits", SPLITS, ids=lambda s: f"S{s}")
def test_tiny_family(case, num_splits):
    case = dict(case)
    w = W.paged_workload(case.pop("seed"), table="pool", slack=0.3, name="tiny", **case)
    kc, vc, ref = _oracle(w)
    c, out = _run(w, num_splits)
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_bits_equal(c.value_cache, vc, "value_cache")
    assert_attention_close(out, ref, f"attention S={num_splits}")


# Prefill-kernel cases: items of 128 / Q tokens, 64-key tiles with ragged tails, block sizes
# that are not powers of two (and not multiples of 4), D 64 and 128, causal and not.
PREFILL = [
    dict(seed=120, past=[0, 150], n_new=[70, 129], num_heads=32, kv_num_heads=8,
         head_size=128, block_size=16),
    dict(seed=121, past=[77], n_new=[200], num_heads=4, kv_num_heads=4, head_size=64,
         block_size=12),                                              # Q = 1: 128-token items
    dict(seed=122, past=[10, 300], n_new=[50, 9], num_heads=6, kv_num_heads=2, head_size=128,
         block_size=5),                                               # Q = 3, bs = 5
    dict(seed=123, past=[40, 0], n_new=[5, 3], num_heads=64, kv_num_heads=1, head_size=64,
         block_size=16),                                              # Q = 64: 2-token items
    dict(seed=124, past=[100], n_new=[40], num_heads=32, kv_num_heads=2, head_size=128,
         block_size=32, causal=0),                                    # Q = 16, not causal
    dict(seed=125, past=[1000, 3], n_new=[300, 1], num_heads=16, kv_num_heads=2,
         head_size=128, block_size=16, packed=True, rotary_mode=W.ROTARY_NEOX,
         rotary_dim=64, rotary_positions=1400),                       # Q = 8, packed, rotary
    dict(seed=126, past=[50, 7], n_new=[70, 33], num_heads=8, kv_num_heads=2, head_size=128,
         block_size=48),                      # bs a multiple of 16, not a power of two: divides
    dict(seed=127, past=[100, 20], n_new=[65, 1], num_heads=4, kv_num_heads=1, head_size=64,
         block_size=24),                      # bs a multiple of 8, not of 16: per-key lookups
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: str(c["seed"]))
def test_prefill_family(case):
    case = dict(case)
    w = W.paged_workload(case.pop("seed"), table="pool", slack=0.2, name="prefill", **case)
    kc, vc, ref = _oracle(w)
    c, out = _run(w)
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_attention_close(out, ref, "prefill")


# Head size 256 and query-head groups above 64 (a kv head with Q > 64, or Q > 16 at D = 256, is
# served as groups of at most 16 query heads that read the same cache head).
WIDE_SHAPES = [
    dict(seed=190, past=[37, 300, 1000], n_new=[1, 1, 1], num_heads=8, kv_num_heads=2,
         head_size=256, block_size=16),                               # decode, Q = 4
    dict(seed=191, past=[0, 150], n_new=[70, 9], num_heads=8, kv_num_heads=8, head_size=256,
         block_size=32),                                              # prefill, Q = 1
    dict(seed=192, past=[100, 12], n_new=[3, 40], num_heads=16, kv_num_heads=2, head_size=256,
         block_size=16, packed=True, rotary_mode=W.ROTARY_NEOX, rotary_dim=256,
         rotary_positions=256),                                       # packed, NeoX on all dims
    dict(seed=193, past=[45, 7], n_new=[2, 33], num_heads=32, kv_num_heads=1, head_size=256,
         block_size=8, rotary_mode=W.ROTARY_INTERLEAVED, rotary_dim=64,
         rotary_positions=128),                                       # Q = 32 -> 2 groups of 16
    dict(seed=194, past=[50], n_new=[20], num_heads=4, kv_num_heads=4, head_size=256,
         block_size=24, causal=0),                                    # bs not a power of two
    dict(seed=195, past=[130, 600], n_new=[1, 1], num_heads=128, kv_num_heads=1,
         head_size=128, block_size=16),                               # decode, Q = 128
    dict(seed=196, past=[40, 0], n_new=[3, 9], num_heads=128, kv_num_heads=1, head_size=64,
         block_size=16),                                              # prefill, Q = 128
    dict(seed=197, past=[70], n_new=[5], num_heads=256, kv_num_heads=2, head_size=128,
         block_size=32, causal=0),                                    # Q = 128, two kv heads
    dict(seed=198, past=[20, 200], n_new=[1, 1], num_heads=96, kv_num_heads=1, head_size=64,
         block_size=16),                                              # Q = 96 -> 6 groups of 16
]


@pytest.mark.parametrize("case", WIDE_SHAPES, ids=lambda c: str(c["seed"]))
@pytest.mark.parametrize("num_splits", [pa.PA_SPLITS_AUTO, pa.PA_SPLITS_PAGE_RULE, 3],
                         ids=lambda s: f"S{s}")
def test_wide_shapes(case, num_splits):
    case = dict(case)
    w = W.paged_workload(case.pop("seed"), table="pool", slack=0.2, name="wide", **case)
    kc, vc, ref = _oracle(w)
    c, out = _run(w, num_splits)
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_bits_equal(c.value_cache, vc, "value_cache")
    assert_attention_close(out, ref, f"wide S={num_splits}")
    c1 = dev.PagedCase(w)
    out1 = c1.append_attention(num_splits)
    torch.cuda.synchronize()
    assert_bits_equal(out1, out, "one-call step")


# Prefill rows whose scores rise by more than 2^8 after the first 64-key tile: the kernel's
# lazily raised maximum rescales O and l (the CPU suite shows the raise occurs in most of these
# columns and that a wrong rescale would exceed the bar).
@pytest.mark.parametrize("case", RAISE_CASES, ids=lambda c: str(c["seed"]))
def test_prefill_max_raise(case):
    case = dict(case)
    w = W.paged_workload(case.pop("seed"), table="pool", slack=0.2, name="raise", **case)
    kc, vc, ref = _oracle(w)
    raised, total = raise_columns(w, kc)
    assert raised > 0.5 * total, (raised, total)
    c, out = _run(w)
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_attention_close(out, ref, "prefill with max raises")


# Fused query rotation: the key/value append plus q_out, each bit-identical to the oracle.
QROT = [
    dict(seed=130, past=[3, 4000, 77, 1], n_new=[1, 1, 1, 1], num_heads=8, kv_num_heads=8,
         head_size=128, block_size=32, rotary_mode=W.ROTARY_NEOX, rotary_dim=128,
         rotary_positions=4096, use_slot_mapping=True),                # NeoX on all dims
    dict(seed=131, past=[3, 900, 77], n_new=[1, 4, 9], num_heads=16, kv_num_heads=8,
         head_size=128, block_size=32, rotary_mode=W.ROTARY_INTERLEAVED, rotary_dim=128,
         rotary_positions=1024),                                      # interleaved pairs
    dict(seed=132, past=[0, 60], n_new=[33, 5], num_heads=32, kv_num_heads=8, head_size=128,
         block_size=16, packed=True, rotary_mode=W.ROTARY_NEOX, rotary_dim=64,
         rotary_positions=128),                                       # NeoX on part of the row
    dict(seed=133, past=[5, 17], n_new=[6, 2], num_heads=6, kv_num_heads=2, head_size=128,
         block_size=16, rotary_mode=W.ROTARY_NEOX, rotary_dim=48, rotary_positions=64),
    dict(seed=134, past=[5, 17], n_new=[6, 2], num_heads=4, kv_num_heads=2, head_size=64,
         block_size=8, packed=True, rotary_mode=W.ROTARY_NEOX, rotary_dim=40,
         rotary_positions=64),                                        # element-wise path
    dict(seed=135, past=[9, 2, 30], n_new=[2, 7, 1], num_heads=8, kv_num_heads=1,
         head_size=64, block_size=16, rotary_mode=W.ROTARY_INTERLEAVED, rotary_dim=36,
         rotary_positions=64),                                        # element-wise, interleaved
    dict(seed=136, past=[12, 0], n_new=[3, 5], num_heads=8, kv_num_heads=2, head_size=128,
         block_size=16, packed=True),                                 # no rotary: copies
    dict(seed=138, past=[5, 17], n_new=[6, 2], num_heads=8, kv_num_heads=2, head_size=256,
         block_size=16, packed=True, rotary_mode=W.ROTARY_NEOX, rotary_dim=256,
         rotary_positions=64),                                        # D = 256
]


@pytest.mark.parametrize("case", QROT, ids=lambda c: str(c["seed"]))
def test_append_rotate_query(case):
    case = dict(case)
    sm = case.pop("use_slot_mapping", False)
    w = W.paged_workload(case.pop("seed"), table="pool", slack=0.2, name="qrot",
                         use_slot_mapping=sm, **case)
    kc, vc = oracle.kv_append(w)
    qref = oracle.rotate_query(w)
    c = dev.PagedCase(w)
    q_out = c.append_rotate_query(use_slot_mapping=sm)
    torch.cuda.synchronize()
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_bits_equal(c.value_cache, vc, "value_cache")
    assert_bits_equal(q_out, qref, "q_out")


def test_append_rotate_query_many_sequences():
    """300 one-token sequences: cu is searched in LDS instead of in lanes, several tokens per
    wave."""
    n = 300
    w = W.paged_workload(137, past=list(range(5, 5 + n)), n_new=[1] * n, num_heads=4,
                         kv_num_heads=2, head_size=64, block_size=16, table="pool", slack=0.1,
                         rotary_mode=W.ROTARY_NEOX, rotary_dim=64, rotary_positions=512,
                         name="qrot_many")
    kc, vc = oracle.kv_append(w)
    qref = oracle.rotate_query(w)
    c = dev.PagedCase(w)
    q_out = c.append_rotate_query()
    torch.cuda.synchronize()
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_bits_equal(q_out, qref, "q_out")


def test_append_rotate_query_mixed_full_size(mixed):
    """The mixed workload (packed rows, NeoX on all dims, derived slots): caches and every rotated
    query row bit-identical; attention over q_out matches the oracle on the rotated rows."""
    w = mixed
    kc, vc = oracle.kv_append(w)
    qref = oracle.rotate_query(w)
    c = dev.PagedCase(w)
    q_out = c.append_rotate_query()
    torch.cuda.synchronize()
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_bits_equal(q_out, qref, "q_out")


# Contiguous BNSH cache append (the append page's own pass): whole caches bit-identical.
BNSH = [
    dict(seed=140, batch=3, seq_len=5, num_heads=4, kv_num_heads=2, head_size=64, max_seq=24,
         key_total=[9, 5, 21]),                                       # no rotary
    dict(seed=141, batch=3, seq_len=7, num_heads=8, kv_num_heads=8, head_size=128,
         max_seq=40, key_total=[12, 3, 30], rotary_mode=W.ROTARY_NEOX),  # past 0 (total < S)
    dict(seed=142, batch=2, seq_len=33, num_heads=32, kv_num_heads=8, head_size=128,
         max_seq=96, key_total=[90, 40], packed=True, rotary_mode=W.ROTARY_NEOX,
         rotary_dim=64),                                             # rows past the cache
    dict(seed=143, batch=4, seq_len=6, num_heads=6, kv_num_heads=2, head_size=128, max_seq=32,
         key_total=[6, 12, 7, 9], total_seq=6, rotary_mode=W.ROTARY_INTERLEAVED),  # prompt
    dict(seed=144, batch=2, seq_len=9, num_heads=4, kv_num_heads=1, head_size=64, max_seq=40,
         key_total=[20, 35], packed=True, rotary_mode=W.ROTARY_NEOX, rotary_dim=40),
    dict(seed=145, batch=2, seq_len=9, num_heads=4, kv_num_heads=2, head_size=64, max_seq=40,
         key_total=[20, 35], rotary_mode=W.ROTARY_INTERLEAVED, rotary_dim=36,
         rotary_positions=30),                                       # rows past the table
    dict(seed=146, batch=2, seq_len=7, num_heads=8, kv_num_heads=4, head_size=256, max_seq=32,
         key_total=[12, 30], rotary_mode=W.ROTARY_NEOX),              # D = 256
]


@pytest.mark.parametrize("case", BNSH, ids=lambda c: str(c["seed"]))
def test_bnsh_append(case):
    case = dict(case)
    bw = W.bnsh_workload(case.pop("seed"), name="bnsh", **case)
    pk, pv = oracle.kv_append_bnsh(bw)
    c = dev.BnshCase(bw)
    gk, gv = c.append()
    torch.cuda.synchronize()
    assert_bits_equal(gk, pk, "present_key")
    assert_bits_equal(gv, pv, "present_value")


def test_bnsh_append_full_size():
    bw = W.bnsh_append()
    pk, pv = oracle.kv_append_bnsh(bw)
    c = dev.BnshCase(bw)
    gk, gv = c.append()
    torch.cuda.synchronize()
    assert_bits_equal(gk, pk, "present_key")
    assert_bits_equal(gv, pv, "present_value")


def test_append_stress_bit_exact():
    """The append bandwidth workload (65536 packed rows, NeoX rotary on all dims): both caches
    bit-identical to the oracle's, every slot."""
    w = W.append_stress()
    kc, vc = oracle.kv_append(w)
    c = dev.PagedCase(w)
    c.append()
    torch.cuda.synchronize()
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_bits_equal(c.value_cache, vc, "value_cache")


@pytest.mark.parametrize("B", [100, 300])
@pytest.mark.parametrize("num_splits", [pa.PA_SPLITS_AUTO, pa.PA_SPLITS_PAGE_RULE, 3],
                         ids=lambda s: f"S{s}")
def test_many_sequences_attention(B, num_splits):
    """More sequences than one planner wave (100) and than one planner chunk (300): one-token
    decodes on varied past lengths, every 37th sequence a 40-token prefill, one empty sequence."""
    def past(r):
        return r.integers(0, 400, size=B)

    def n_new(r):
        n = np.ones(B, dtype=np.int64)
        n[::37] = 40
        n[B // 2] = 0
        return n

    w = W.paged_workload(150 + B, past=past, n_new=n_new, num_heads=8, kv_num_heads=2,
                         head_size=64, block_size=16, table="pool", name=f"many{B}")
    kc, vc, ref = _oracle(w)
    c, out = _run(w, num_splits)
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_attention_close(out, ref, f"B={B}")


@pytest.mark.parametrize("one_call", [False, True], ids=["two_calls", "one_call"])
@pytest.mark.parametrize("num_splits", [pa.PA_SPLITS_AUTO, 3], ids=lambda s: f"S{s}")
@pytest.mark.parametrize("kv_heads", [2, 8], ids=["serial", "fused"])
def test_graph_capture_replays_match_eager(num_splits, one_call, kv_heads):
    """The append and the attention (two calls, or pa_append_attention) captured into one HIP
    graph (the library enqueues kernels only: no allocation, memset or synchronization): every
    replay, with eager library work between replays, is bit-identical to the eager step. With 8
    kv heads the decode and prefill items share one launch (the merge of split rows follows in a
    launch of its own); with 2 the decode kernel runs alone, then the prefill launch."""
    w = W.paged_workload(160, past=[40, 300, 5, 1000], n_new=[1, 70, 1, 33],
                         num_heads=4 * kv_heads, kv_num_heads=kv_heads, head_size=128,
                         block_size=16, table="pool", name="graph")
    c = dev.PagedCase(w)

    def step():
        if one_call:
            c.append_attention(num_splits)
        else:
            c.append()
            c.attention(num_splits)

    c.append()
    ref = c.attention(num_splits).clone()  # eager; also sizes the workspace outside the graph
    torch.cuda.synchronize()
    kc_ref, vc_ref = c.key_cache.clone(), c.value_cache.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        c.output.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(c.output, ref, f"replay {i}")
        assert_bits_equal(c.key_cache, kc_ref, f"key_cache after replay {i}")
        assert_bits_equal(c.value_cache, vc_ref, f"value_cache after replay {i}")
        eager = c.attention(num_splits, out=torch.empty_like(ref))
        torch.cuda.synchronize()
        assert_bits_equal(eager, ref, f"eager after replay {i}")


# pa_append_attention against the two separate calls on fresh copies of the same workload:
# caches and output bit for bit, and the output against the oracle.
APPEND_ATTN = [TINY[1], TINY[3], TINY[4], TINY[5], PREFILL[0], PREFILL[5], PREFILL[7]]


@pytest.mark.parametrize("case", APPEND_ATTN, ids=lambda c: str(c["seed"]))
@pytest.mark.parametrize("num_splits", [pa.PA_SPLITS_AUTO, pa.PA_SPLITS_PAGE_RULE, 3],
                         ids=lambda s: f"S{s}")
def test_append_attention_matches_separate_calls(case, num_splits):
    case = dict(case)
    w = W.paged_workload(case.pop("seed"), table="pool", slack=0.2, name="append_attn", **case)
    kc, vc, ref = _oracle(w)
    sep, out_sep = _run(w, num_splits)
    c = dev.PagedCase(w)
    out = c.append_attention(num_splits)
    torch.cuda.synchronize()
    assert_bits_equal(c.key_cache, sep.key_cache, "key_cache")
    assert_bits_equal(c.value_cache, sep.value_cache, "value_cache")
    assert_bits_equal(out, out_sep, "output")
    assert_bits_equal(c.key_cache, kc, "key_cache vs oracle")
    assert_attention_close(out, ref, f"append_attention S={num_splits}")


@pytest.mark.parametrize("B", [100, 300])
def test_append_attention_many_sequences(B):
    """Past the one-wave planner (100 sequences) and past one planner chunk and the lane-held
    cumulative lengths of the append (300): the planner workgroup runs with 256 threads."""
    def past(r):
        return r.integers(0, 400, size=B)

    def n_new(r):
        n = np.ones(B, dtype=np.int64)
        n[::37] = 40
        n[B // 2] = 0
        return n

    w = W.paged_workload(170 + B, past=past, n_new=n_new, num_heads=8, kv_num_heads=2,
                         head_size=64, block_size=16, table="pool", name=f"append_attn{B}")
    kc, vc, ref = _oracle(w)
    sep, out_sep = _run(w)
    c = dev.PagedCase(w)
    out = c.append_attention()
    torch.cuda.synchronize()
    assert_bits_equal(c.key_cache, sep.key_cache, "key_cache")
    assert_bits_equal(c.value_cache, sep.value_cache, "value_cache")
    assert_bits_equal(out, out_sep, "output")
    assert_attention_close(out, ref, f"B={B}")


@pytest.mark.parametrize("case", [QROT[0], QROT[2], QROT[4]], ids=lambda c: str(c["seed"]))
def test_append_attention_rotates_query(case):
    """With q_out: the rotated rows bit-identical to the oracle's, and the output bit-identical
    to pa_kv_append_rotate_query followed by attention over q_out."""
    case = dict(case)
    sm = case.pop("use_slot_mapping", False)
    w = W.paged_workload(case.pop("seed"), table="pool", slack=0.2, name="append_attn_q",
                         use_slot_mapping=sm, **case)
    qref = oracle.rotate_query(w)
    sep = dev.PagedCase(w)
    q_sep = sep.append_rotate_query(use_slot_mapping=sm)
    shape = pa.paged_shape(w["B"], w["T"], w["H"], w["G"], w["D"], w["NB"], w["bs"], w["MB"],
                           False)
    ws, n = sep.workspace_for(pa.PA_SPLITS_AUTO)
    out_sep = torch.empty_like(sep.output)
    pa.pa_paged_attention(shape, q_sep, sep.key_cache, sep.value_cache, sep.cu, sep.past,
                          sep.block_table, w["scale"], w["causal"], pa.PA_SPLITS_AUTO, ws, n,
                          out_sep)
    c = dev.PagedCase(w)
    q_out = torch.empty_like(q_sep)
    out = c.append_attention(q_out=q_out, use_slot_mapping=sm)
    torch.cuda.synchronize()
    assert_bits_equal(q_out, qref, "q_out")
    assert_bits_equal(c.key_cache, sep.key_cache, "key_cache")
    assert_bits_equal(c.value_cache, sep.value_cache, "value_cache")
    assert_bits_equal(out, out_sep, "output")


def test_append_attention_gqa_full_size(gqa):
    """The batch-64 serving decode through the one-call path: caches bit-exact against the
    oracle, output within the attention bar."""
    w, kc, vc, ref = gqa
    c = dev.PagedCase(w)
    out = c.append_attention(pa.PA_SPLITS_AUTO)
    torch.cuda.synchronize()
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_bits_equal(c.value_cache, vc, "value_cache")
    assert_attention_close(out, ref, "append_attention gqa")


@pytest.mark.parametrize("causal", [0, 1])
def test_non_causal_and_prefill(causal):
    w = W.paged_workload(110, past=[3, 60, 0], n_new=[33, 1, 17], num_heads=8, kv_num_heads=2,
                         head_size=128, block_size=16, table="pool", causal=causal,
                         name="causal")
    kc, vc, ref = _oracle(w)
    _, out = _run(w)
    assert_attention_close(out, ref, f"causal={causal}")


def test_tiny_decode_workload():
    w = W.tiny_decode()
    kc, vc, ref = _oracle(w)
    c, out = _run(w, pa.PA_SPLITS_PAGE_RULE)
    assert_bits_equal(c.key_cache, kc)
    assert_bits_equal(c.value_cache, vc)
    assert_attention_close(out, ref)


@pytest.mark.parametrize("mode", [W.ROTARY_NEOX, W.ROTARY_INTERLEAVED])
@pytest.mark.parametrize("use_slot_mapping", [True, False])
def test_rotary_append_decode(mode, use_slot_mapping):
    w = W.rotary_append_decode(rotary_mode=mode)
    kc, vc, ref = _oracle(w)
    c, out = _run(w, pa.PA_SPLITS_PAGE_RULE, use_slot_mapping=use_slot_mapping)
    g = c.key_cache.cpu().numpy()
    assert np.abs(g.astype(np.float32) - kc.astype(np.float32)).max() <= ROT_ABS
    assert_bits_equal(g, kc, "rotated key_cache")       # matched float32 arithmetic
    assert_bits_equal(c.value_cache, vc, "value_cache")
    assert_attention_close(out, ref)


def test_nan_in_stale_rows_never_reaches_output():
    w = W.paged_workload(111, past=[70, 5, 129], n_new=[1, 12, 1], num_heads=8, kv_num_heads=2,
                         head_size=128, block_size=16, table="pool", slack=0.5, poison=True,
                         name="poison")
    kc, vc, ref = _oracle(w)
    for s in (pa.PA_SPLITS_AUTO, 4):
        _, out = _run(w, s)
        assert_attention_close(out, ref, f"poisoned S={s}")


def test_page_permutation_is_bit_identical():
    w = W.paged_workload(112, past=[300, 41], n_new=[1, 20], num_heads=8, kv_num_heads=2,
                         head_size=128, block_size=16, table="pool", name="perm")
    _, a = _run(w)
    a = a.cpu().numpy()
    perm = np.random.default_rng(3).permutation(w["NB"])
    inv = np.argsort(perm)
    w2 = dict(w)
    w2["key_cache"], w2["value_cache"] = w["key_cache"][perm], w["value_cache"][perm]
    bt = w["block_table"].copy()
    bt[bt >= 0] = inv[bt[bt >= 0]]
    w2["block_table"] = bt
    _, b = _run(w2)
    assert_bits_equal(b, a, "permuted pages")


@pytest.fixture(scope="module")
def gqa():
    w = W.gqa_decode()
    kc, vc, ref = _oracle(w)
    return w, kc, vc, ref


@pytest.mark.parametrize("num_splits", SPLITS + [7], ids=lambda s: f"S{s}")
def test_gqa_serving_decode_full_size(gqa, num_splits):
    w, kc, vc, ref = gqa
    c, out = _run(w, num_splits)
    if num_splits == pa.PA_SPLITS_AUTO:
        assert_bits_equal(c.key_cache, kc, "key_cache")
        assert_bits_equal(c.value_cache, vc, "value_cache")
    assert_attention_close(out, ref, f"S={num_splits}")


@pytest.fixture(scope="module")
def mixed():
    return W.mixed_prefill_decode()


def test_mixed_prefill_decode_full_size(mixed):
    w = mixed
    c = dev.PagedCase(w)
    c.append()
    out = c.attention(pa.PA_SPLITS_AUTO).cpu().numpy()
    torch.cuda.synchronize()
    # the append over the whole cache, bit for bit
    kc, vc = oracle.kv_append(w)
    assert_bits_equal(c.key_cache, kc, "key_cache")
    assert_bits_equal(c.value_cache, vc, "value_cache")
    # attention on every row: the 4096 prefill rows and the 56 decode rows, each computed by the
    # oracle as the equivalent one-token decode, on host threads
    ref = oracle_rows(oracle, w, kc, vc)
    assert_attention_close(out, ref, "mixed, every row")


# ------------------------------------------------------------------ combine of oracle partials
@pytest.mark.parametrize("S", [2, 5])
@pytest.mark.parametrize("out_dtype", [pa.PA_F16, pa.PA_F32])
def test_combine_uniform_splits(S, out_dtype):
    w = W.paged_workload(120, past=[333, 70, 1000], n_new=[1, 1, 1], num_heads=8,
                         kv_num_heads=2, head_size=128, block_size=16, name="comb")
    o, m, l = oracle.paged_attention_partials(w, S)
    ref = oracle.split_combine(o, m, l, lanes=w["H"], head_dim=128, num_splits=S,
                               out_dtype=np.float16 if out_dtype == pa.PA_F16 else np.float32)
    got = dev.combine(o, m, l, lanes=w["H"], head_dim=128, num_splits=S, out_dtype=out_dtype)
    torch.cuda.synchronize()
    if out_dtype == pa.PA_F16:
        assert_attention_close(got, ref)
    else:
        g = got.cpu().numpy()
        assert np.allclose(g, ref, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("lanes", [1, 3, 5, 7, 12, 33])
@pytest.mark.parametrize("uniform", [0, 3], ids=["csr", "uniform3"])
def test_combine_row_blocks(D, lanes, uniform):
    """Random partial sets over both merge layouts: one row block of 256/D rows per wave, or two
    when a group has that many rows (lanes >= 8 at D = 64, >= 4 at D = 128), with ragged last
    blocks, empty groups and empty partials, in CSR and uniform-split form."""
    rp = W.random_partials(200 + lanes + D + uniform, groups=37, lanes=lanes, head_dim=D,
                           uniform_splits=uniform)
    kw = dict(lanes=lanes, head_dim=D)
    if uniform:
        kw.update(num_splits=uniform)
    else:
        kw.update(group_ptr=rp["group_ptr"])
    ref = oracle.split_combine(rp["o"], rp["m"], rp["l"], out_dtype=np.float32, **kw)
    got = dev.combine(rp["o"], rp["m"], rp["l"], out_dtype=pa.PA_F32, **kw).cpu().numpy()
    torch.cuda.synchronize()
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-6), float(np.abs(got - ref).max())
    ref16 = oracle.split_combine(rp["o"], rp["m"], rp["l"], out_dtype=np.float16, **kw)
    got16 = dev.combine(rp["o"], rp["m"], rp["l"], out_dtype=pa.PA_F16, **kw)
    torch.cuda.synchronize()
    assert_attention_close(got16, ref16, f"combine fp16 lanes={lanes} D={D}")


def test_combine_csr_with_empty_and_sentinel_groups():
    w = W.paged_workload(121, past=[90, 20], n_new=[1, 1], num_heads=4, kv_num_heads=4,
                         head_size=64, block_size=16, name="comb")
    o, m, l = oracle.paged_attention_partials(w, 4, chunk_keys=32)   # 91 keys: 3 + 1 empty
    # groups: token 0's 4 units, an empty group, token 1's 4 units in reverse order
    order = np.r_[0, 1, 2, 3, 7, 6, 5, 4]
    H, D = w["H"], w["D"]
    o2 = o.reshape(8, H, D)[order].reshape(-1, D)
    m2 = m.reshape(8, H)[order].reshape(-1)
    l2 = l.reshape(8, H)[order].reshape(-1)
    gp = np.array([0, 4, 4, 8], dtype=np.int32)
    ref = oracle.split_combine(o2, m2, l2, lanes=H, head_dim=D, group_ptr=gp,
                               out_dtype=np.float32)
    got = dev.combine(o2, m2, l2, lanes=H, head_dim=D, group_ptr=gp, out_dtype=pa.PA_F32)
    g = got.cpu().numpy()
    assert np.all(g[H:2 * H] == 0)
    assert np.allclose(g, ref, rtol=1e-5, atol=1e-6)
