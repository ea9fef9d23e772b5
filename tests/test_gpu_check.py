"""GPU tests of pa_check_paged_indices against the plain statement of the index rules
(tests/index_rules.py): seeded workloads pass every rule, each hand-made violation raises its
bits, and seeded random corruptions of a rotary workload give the same flag word on both sides.
The check only reads the index arrays, so corrupted contents are safe to pass to it. Duplicate
written slots (two rows, one slot: the append would race) are checked within and across 256-row
tiles."""
import copy

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_gqa_paged_amd as pa  # noqa: E402
from block_sparse_gqa_paged_amd import device as dev  # noqa: E402
from block_sparse_gqa_paged_amd import workloads as W  # noqa: E402
from index_rules import expected_flags, workload_flags  # noqa: E402

pytestmark = pytest.mark.gpu

CU_BITS = pa.PA_CHECK_CU_START | pa.PA_CHECK_CU_ORDER | pa.PA_CHECK_CU_END


def _device_flags(cu, past, bt, slot, *, T, NB, bs, MB, rotary_positions=0, B=None):
    B = len(past) if B is None else B
    shape = pa.paged_shape(B, T, 4, 2, 64, NB, bs, MB, False)
    t = lambda a: None if a is None else torch.tensor(np.asarray(a, np.int32), device="cuda")
    flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    pa.pa_check_paged_indices(shape, t(cu), t(past), t(bt), t(slot), flags,
                              rotary_positions=rotary_positions)
    torch.cuda.synchronize()
    return int(flags.item())


@pytest.mark.parametrize("name", ["tiny", "rot_neox", "rot_inter", "gqa", "mixed"])
@pytest.mark.parametrize("slot,table", [(True, True), (False, True), (True, False)])
def test_seeded_workloads_pass(name, slot, table):
    w = {"tiny": W.tiny_decode, "gqa": W.gqa_decode, "mixed": W.mixed_prefill_decode,
         "rot_neox": lambda: W.rotary_append_decode(rotary_mode=W.ROTARY_NEOX),
         "rot_inter": lambda: W.rotary_append_decode(rotary_mode=W.ROTARY_INTERLEAVED)}[name]()
    if slot and w["slot_mapping"] is None:
        pytest.skip("workload derives its slots from the block table")
    c = dev.PagedCase(w)
    got = c.check_indices(use_slot_mapping=slot, use_block_table=table)
    assert got == workload_flags(w, use_slot_mapping=slot, use_block_table=table) == 0


def _base():
    return dict(cu=[0, 2, 5], past=[5, 0], bt=[[3, 6, -1], [1, 0, -1]],
                slot=[25, 26, 4, 5, 6], T=5, NB=8, bs=4, MB=3, rotary_positions=16)


EDITS = [
    ("none", lambda d: None),
    ("cu_end", lambda d: d["cu"].__setitem__(2, 6)),
    ("cu_start", lambda d: d["cu"].__setitem__(0, 1)),
    ("cu_order", lambda d: d.update(cu=[0, 4, 3], T=3, slot=[25, 26, 4])),
    ("past", lambda d: d["past"].__setitem__(1, -1)),
    ("width", lambda d: d.update(past=[11, 0], bt=[[3, 6, 2], [1, 0, -1]], slot=None)),
    ("entry_high", lambda d: d["bt"][1].__setitem__(0, 8)),
    ("entry_neg", lambda d: d["bt"][0].__setitem__(0, -1)),
    ("entry_unused", lambda d: d["bt"][0].__setitem__(2, 99)),
    ("slot_high", lambda d: d["slot"].__setitem__(4, 32)),
    ("slot_mismatch", lambda d: d["slot"].__setitem__(4, 7)),
    ("slot_skip", lambda d: d["slot"].__setitem__(0, -1)),
    ("position", lambda d: d.__setitem__("rotary_positions", 6)),
    ("no_table", lambda d: d.update(bt=None)),
    ("slot_dup", lambda d: d["slot"].__setitem__(4, 25)),            # rows 0 and 4 share a slot
    ("slot_dup_derived", lambda d: d.update(slot=None, bt=[[3, 6, -1], [6, 0, -1]])),  # shared block
]


def test_duplicate_slot_across_tiles():
    """600 new rows (three 256-row tiles): distinct slots pass; one repeated slot between the
    first and the last tile raises the duplicate bit, on both sides."""
    T, bs, NB = 600, 16, 64
    cu, past = [0, 200, 450, T], [0, 7, 30]
    slot = list(np.random.default_rng(5).permutation(NB * bs)[:T])
    kw = dict(T=T, NB=NB, bs=bs, MB=64)
    assert _device_flags(cu, past, None, slot, **kw) == expected_flags(cu, past, None, slot,
                                                                     **kw) == 0
    slot[590] = slot[3]
    want = expected_flags(cu, past, None, slot, **kw)
    assert want == pa.PA_CHECK_SLOT_DUP
    assert _device_flags(cu, past, None, slot, **kw) == want


@pytest.mark.parametrize("name,edit", EDITS, ids=[e[0] for e in EDITS])
def test_hand_made_violations(name, edit):
    d = copy.deepcopy(_base())
    edit(d)
    want = expected_flags(d["cu"], d["past"], d["bt"], d["slot"], T=d["T"], NB=d["NB"],
                          bs=d["bs"], MB=d["MB"], rotary_positions=d["rotary_positions"])
    got = _device_flags(d["cu"], d["past"], d["bt"], d["slot"], T=d["T"], NB=d["NB"],
                        bs=d["bs"], MB=d["MB"], rotary_positions=d["rotary_positions"])
    if want & (pa.PA_CHECK_CU_START | pa.PA_CHECK_CU_ORDER):
        assert got & CU_BITS == want & CU_BITS  # rows have no defined sequence
    else:
        assert got == want
    assert (name == "none" or name.endswith(("unused", "skip")) or name == "no_table") == \
        (got == 0)


@pytest.mark.parametrize("seed", range(6))
def test_random_corruptions_of_a_rotary_workload(seed):
    w = W.rotary_append_decode(rotary_mode=W.ROTARY_NEOX)
    rng = np.random.default_rng(1000 + seed)
    cu, past = w["cu"].copy(), w["past"].copy()
    bt, slot = w["block_table"].copy(), w["slot_mapping"].copy()
    B, T, MB, NB, bs = w["B"], w["T"], w["MB"], w["NB"], w["bs"]
    for _ in range(rng.integers(1, 4)):
        kind = rng.integers(0, 5)
        if kind == 0:
            past[rng.integers(B)] = rng.integers(-3, 5000)
        elif kind == 1:
            bt[rng.integers(B), rng.integers(MB)] = rng.integers(-2, NB + 3)
        elif kind == 2:
            slot[rng.integers(T)] = rng.integers(-2, NB * bs + 3)
        elif kind == 3:
            cu[rng.integers(1, B + 1)] = rng.integers(0, T + 2)
        else:
            b = rng.integers(B)  # a valid table entry moved: slots of that block disagree
            j = (past[b]) // bs
            if j < MB:
                bt[b, j] = (bt[b, j] + 1) % NB
    rot = w["cos"].shape[0]
    want = expected_flags(cu, past, bt, slot, T=T, NB=NB, bs=bs, MB=MB, rotary_positions=rot)
    got = _device_flags(cu, past, bt, slot, T=T, NB=NB, bs=bs, MB=MB, rotary_positions=rot)
    if want & (pa.PA_CHECK_CU_START | pa.PA_CHECK_CU_ORDER):
        assert got & CU_BITS == want & CU_BITS
    else:
        assert got == want
