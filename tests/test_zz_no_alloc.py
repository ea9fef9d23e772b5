"""GPU check of pa_paged_attention_noalloc (the entry point whose scratch is the library's static
device array): on consecutive calls, the second with a smaller input, its output equals
pa_paged_attention's with a workspace of the caller's, bit for bit, and the oracle's within the
attention bar; captured into a HIP graph, every replay equals the eager result."""
import pytest

torch = pytest.importorskip("torch")

import block_sparse_gqa_paged_amd as pa  # noqa: E402
import oracle  # noqa: E402
from block_sparse_gqa_paged_amd import device as dev  # noqa: E402
from block_sparse_gqa_paged_amd import workloads as W  # noqa: E402
from parity import assert_attention_close, assert_bits_equal  # noqa: E402

pytestmark = pytest.mark.gpu


def _noalloc(c, num_splits):
    w = c.w
    out = torch.full_like(c.output, float("nan"))
    pa.pa_paged_attention_noalloc(c.shape, c.query, c.key_cache, c.value_cache, c.cu, c.past,
                                  c.block_table, w["scale"], w["causal"], num_splits, out)
    return out


# a larger call (split decode rows with long contexts, prefill rows, every split policy's
# partials), then smaller ones: whatever the earlier call left in the array must not matter
CASES = [
    dict(seed=300, past=[3000, 40, 700, 1500], n_new=[1, 70, 1, 1], num_heads=32,
         kv_num_heads=8, head_size=128, block_size=16),
    dict(seed=301, past=[37, 100], n_new=[1, 1], num_heads=4, kv_num_heads=2, head_size=64,
         block_size=16),
]


@pytest.mark.parametrize("num_splits", [pa.PA_SPLITS_AUTO, pa.PA_SPLITS_PAGE_RULE, 3],
                         ids=lambda s: f"S{s}")
def test_noalloc_matches_workspace_entry_on_consecutive_calls(num_splits):
    cases = []
    for case in CASES:
        case = dict(case)
        w = W.paged_workload(case.pop("seed"), table="pool", slack=0.2, name="noalloc", **case)
        c = dev.PagedCase(w)
        c.append()
        cases.append(c)
    torch.cuda.synchronize()
    outs = [_noalloc(c, num_splits) for c in cases]  # back to back on one stream
    torch.cuda.synchronize()
    for k, (c, out) in enumerate(zip(cases, outs)):
        ref = c.attention(num_splits, out=torch.empty_like(c.output))
        torch.cuda.synchronize()
        assert_bits_equal(out, ref, f"call {k}: noalloc vs workspace entry")
        kc, vc = oracle.kv_append(c.w)
        assert_attention_close(out, oracle.paged_attention(c.w, kc, vc), f"call {k} vs oracle")
    # the larger case again, after the smaller one ran last in the array
    again = _noalloc(cases[0], num_splits)
    torch.cuda.synchronize()
    assert_bits_equal(again, outs[0], "larger case after the smaller one")



@pytest.mark.parametrize("num_splits", [pa.PA_SPLITS_AUTO, 3], ids=lambda s: f"S{s}")
def test_noalloc_graph_replays_match_eager(num_splits):
    """The no-allocation entry captured into a HIP graph (its scratch address looked up by an
    eager call first): every replay is bit-identical to the eager result, also after an eager
    call of another shape has overwritten the shared scratch between replays."""
    cs = []
    for case in CASES:
        case = dict(case)
        w = W.paged_workload(case.pop("seed"), table="pool", slack=0.2, name="noalloc", **case)
        c = dev.PagedCase(w)
        c.append()
        cs.append(c)
    big, small = cs
    torch.cuda.synchronize()
    ref = _noalloc(big, num_splits)
    ref_small = _noalloc(small, num_splits)
    torch.cuda.synchronize()
    out = torch.empty_like(big.output)
    w = big.w

    def call():
        pa.pa_paged_attention_noalloc(big.shape, big.query, big.key_cache, big.value_cache,
                                      big.cu, big.past, big.block_table, w["scale"], w["causal"],
                                      num_splits, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(out, ref, f"replay {i}")
        other = _noalloc(small, num_splits)  # eager, same scratch, another shape
        torch.cuda.synchronize()
        assert_bits_equal(other, ref_small, f"eager smaller call after replay {i}")
