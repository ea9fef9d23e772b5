"""CPU pins of the paged index rules (tests/index_rules.py), the reference of
pa_check_paged_indices: every seeded paged workload satisfies them, and each hand-made violation
raises exactly its own bit."""
import copy

import numpy as np
import pytest

import block_sparse_gqa_paged_amd as pa
from block_sparse_gqa_paged_amd import workloads as W
from index_rules import expected_flags, workload_flags

SMALL = [W.tiny_decode, lambda: W.rotary_append_decode(rotary_mode=W.ROTARY_NEOX),
         lambda: W.rotary_append_decode(rotary_mode=W.ROTARY_INTERLEAVED)]


@pytest.mark.parametrize("make", SMALL, ids=["tiny", "rot_neox", "rot_inter"])
def test_seeded_workloads_satisfy_every_rule(make):
    w = make()
    assert workload_flags(w) == 0
    assert workload_flags(w, use_slot_mapping=False, use_block_table=False) == 0


def _base():
    # 2 sequences, block size 4, 8 blocks, table width 3: past {5, 0}, new {2, 3}
    return dict(cu=[0, 2, 5], past=[5, 0],
                block_table=[[3, 6, -1], [1, 0, -1]],
                slot_mapping=[6 * 4 + 1, 6 * 4 + 2, 1 * 4 + 0, 1 * 4 + 1, 1 * 4 + 2],
                T=5, NB=8, bs=4, MB=3, rotary_positions=16)


def _flags(d):
    d = dict(d)
    return expected_flags(d.pop("cu"), d.pop("past"), d.pop("block_table"),
                          d.pop("slot_mapping"), **d)


def test_hand_made_case_is_valid():
    assert _flags(_base()) == 0


@pytest.mark.parametrize("edit,bit", [
    (lambda d: d["cu"].__setitem__(2, 6), pa.PA_CHECK_CU_END),
    # a negative past length also moves the sequence's rows off their positions and slots
    (lambda d: d["past"].__setitem__(1, -1),
     pa.PA_CHECK_PAST | pa.PA_CHECK_POSITION | pa.PA_CHECK_SLOT_TABLE),
    # 13 keys need 4 blocks of 4, the table holds 3 (all valid; no slot mapping to compare)
    (lambda d: d.update(past=[11, 0], block_table=[[3, 6, 2], [1, 0, -1]], slot_mapping=None),
     pa.PA_CHECK_TABLE_WIDTH),
    (lambda d: d["block_table"][1].__setitem__(0, 8), pa.PA_CHECK_TABLE_ENTRY | pa.PA_CHECK_SLOT_TABLE),
    (lambda d: d["block_table"][0].__setitem__(0, -1), pa.PA_CHECK_TABLE_ENTRY),
    (lambda d: d["block_table"][0].__setitem__(2, 99), 0),              # past the keys: not read
    (lambda d: d["slot_mapping"].__setitem__(4, 32), pa.PA_CHECK_SLOT),
    (lambda d: d["slot_mapping"].__setitem__(4, 7), pa.PA_CHECK_SLOT_TABLE),
    (lambda d: d["slot_mapping"].__setitem__(0, -1), 0),                # not written: allowed
    (lambda d: d.__setitem__("rotary_positions", 6), pa.PA_CHECK_POSITION),
    # row 4 maps to row 0's slot (and off the slot its position has): two rows, one slot
    (lambda d: d["slot_mapping"].__setitem__(4, 25),
     pa.PA_CHECK_SLOT_DUP | pa.PA_CHECK_SLOT_TABLE),
    # derived slots: both sequences' tables name block 6 where their new rows land
    (lambda d: d.update(slot_mapping=None, block_table=[[3, 6, -1], [6, 0, -1]]),
     pa.PA_CHECK_SLOT_DUP),
])
def test_each_violation_raises_its_bit(edit, bit):
    d = copy.deepcopy(_base())
    edit(d)
    assert _flags(d) == bit


def test_disordered_offsets():
    d = copy.deepcopy(_base())
    d["cu"] = [0, 4, 3]
    d["T"] = 3
    assert _flags(d) & pa.PA_CHECK_CU_ORDER
    d = copy.deepcopy(_base())
    d["cu"] = [1, 2, 5]
    assert _flags(d) & pa.PA_CHECK_CU_START
