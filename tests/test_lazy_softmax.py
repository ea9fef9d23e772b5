"""CPU checks of the prefill max-raise inputs: in every case most prefill columns raise their
running maximum after the first 64-key tile (so the kernel's rescale branch runs on the GPU),
and a float64 model of the lazy scheme reproduces the oracle within the attention bar while each
planted rescale mistake (O not rescaled, l not rescaled, alpha doubled) exceeds it."""
import numpy as np
import pytest

import oracle
from block_sparse_gqa_paged_amd import workloads as W
from lazy_softmax import RAISE_CASES, lazy_attention, raise_columns
from parity import ATT_ABS, ATT_REL


def _workload(case):
    case = dict(case)
    return W.paged_workload(case.pop("seed"), table="pool", slack=0.2, name="raise", **case)


@pytest.mark.parametrize("case", RAISE_CASES, ids=lambda c: str(c["seed"]))
def test_raise_occurs_in_most_prefill_columns(case):
    w = _workload(case)
    kc, _ = oracle.kv_append(w)
    raised, total = raise_columns(w, kc)
    assert total > 0 and raised > 0.5 * total, (raised, total)


@pytest.mark.parametrize("case", [RAISE_CASES[0], RAISE_CASES[3], RAISE_CASES[5]],
                         ids=lambda c: str(c["seed"]))
def test_planted_rescale_mistakes_exceed_the_bar(case):
    w = _workload(case)
    kc, vc = oracle.kv_append(w)
    ref = oracle.paged_attention(w, kc, vc).astype(np.float64)

    def excess(mistake):
        rows, out = lazy_attention(w, kc, vc, mistake)
        r = ref[rows]
        return (np.abs(out - r) - (ATT_ABS + ATT_REL * np.abs(r))).max()

    assert excess(None) <= 0
    for mistake in ("no_o_rescale", "no_l_rescale", "alpha_x2"):
        assert excess(mistake) > 0, mistake
