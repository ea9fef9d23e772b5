"""The index contract of the paged calls, stated rule by rule in plain Python: the reference for
pa_check_paged_indices. Rules follow the PagedAttention manifest's inputs (row offsets,
past lengths, block table, slot mapping) and its derived sizes; each returns the PA_CHECK_* bit
of include/pa.h. Rows are mapped to sequences only when the offsets are valid (with disordered
offsets a row's sequence is not defined, and callers compare the offset bits only)."""
import block_sparse_gqa_paged_amd as pa


def expected_flags(cu, past, block_table, slot_mapping, *, T, NB, bs, MB, rotary_positions=0):
    B = len(past)
    cu = [int(x) for x in cu]
    past = [int(x) for x in past]
    bits = 0
    if cu[0] != 0:
        bits |= pa.PA_CHECK_CU_START
    if any(cu[b + 1] < cu[b] for b in range(B)):
        bits |= pa.PA_CHECK_CU_ORDER
    if cu[B] != T:
        bits |= pa.PA_CHECK_CU_END
    if any(p < 0 for p in past):
        bits |= pa.PA_CHECK_PAST
    for b in range(B):
        n = cu[b + 1] - cu[b]
        if n < 0 or past[b] < 0:
            continue
        L = past[b] + n
        if -(-L // bs) > MB:
            bits |= pa.PA_CHECK_TABLE_WIDTH
        if block_table is not None:
            for j in range(MB):
                if j * bs >= L:
                    break
                e = int(block_table[b][j])
                if e < 0 or e >= NB:
                    bits |= pa.PA_CHECK_TABLE_ENTRY
    if bits & (pa.PA_CHECK_CU_START | pa.PA_CHECK_CU_ORDER):
        return bits  # rows have no defined sequence: the remaining rules are not compared
    written = set()  # slots the new rows write, for the duplicate rule
    for i in range(T):
        b = max(k for k in range(B) if cu[k] <= i)
        pos = past[b] + i - cu[b]
        if rotary_positions > 0 and not (0 <= pos < rotary_positions):
            bits |= pa.PA_CHECK_POSITION
        derived = None
        if block_table is not None and pos >= 0 and pos // bs < MB:
            derived = int(block_table[b][pos // bs]) * bs + pos % bs
        s = int(slot_mapping[i]) if slot_mapping is not None else derived
        if s is not None and s >= 0:
            if s in written:
                bits |= pa.PA_CHECK_SLOT_DUP  # two rows write one slot: the append races
            written.add(s)
        if slot_mapping is None or s < 0:
            continue
        if s >= NB * bs:
            bits |= pa.PA_CHECK_SLOT
        elif derived is not None and derived != s:
            bits |= pa.PA_CHECK_SLOT_TABLE
    return bits


def workload_flags(w, *, use_slot_mapping=True, use_block_table=True):
    rot = 0 if w.get("cos") is None else w["cos"].shape[0]
    return expected_flags(w["cu"], w["past"], w["block_table"] if use_block_table else None,
                          w["slot_mapping"] if use_slot_mapping else None, T=w["T"], NB=w["NB"],
                          bs=w["bs"], MB=w["MB"], rotary_positions=rot)
