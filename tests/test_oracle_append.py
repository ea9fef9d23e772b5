"""Pins of the oracle's KV append (rotary + scatter) and of the padded-batch past-length rule.

Page: com.microsoft.SparseAttention "sparse-kv-append.wgsl.jinja" (past-length macro, rotary
macros, main) and the PagedAttention manifest (ScatterKV pass, slot_mapping input).
"""
import numpy as np
import pytest

from block_sparse_gqa_paged_amd import workloads as W


# ------------------------------------------------------------------ past length (padded rule)
@pytest.mark.parametrize("total_scalar,key_total,seq_len,expect", [
    (7, 7, 7, 0),      # prompt mode: scalar total equals the new-token count
    (7, 3, 7, 0),      # prompt mode wins over a padded row's own total
    (7, 100, 7, 0),
    (12, 12, 4, 8),    # history = own total - new tokens
    (12, 5, 4, 1),
    (12, 4, 4, 0),
    (12, 2, 4, 0),     # own total below the new-token count clamps to 0
])
def test_past_length_padded(oracle, total_scalar, key_total, seq_len, expect):
    assert oracle.past_length_padded(total_scalar, key_total, seq_len) == expect


# ------------------------------------------------------------------ scatter without rotary
def _small(seed, **kw):
    args = dict(past=[5, 0, 33], n_new=[3, 17, 1], num_heads=4, kv_num_heads=2, head_size=64,
                block_size=16, table="pool", slack=0.5, name="small")
    args.update(kw)
    return W.paged_workload(seed, **args)


def _identity_table(w):
    """Rewrite w so block b*MB + j holds sequence b's j-th block (contiguous per sequence)."""
    w = dict(w)
    B, MB = w["B"], w["MB"]
    nb = B * MB
    shp = (nb,) + w["key_cache"].shape[1:]
    rng = np.random.default_rng(99)
    w["key_cache"] = rng.standard_normal(shp).astype(np.float16)
    w["value_cache"] = rng.standard_normal(shp).astype(np.float16)
    w["block_table"] = np.arange(nb, dtype=np.int32).reshape(B, MB)
    w["NB"] = nb
    w["slot_mapping"] = None
    return w


@pytest.mark.parametrize("packed", [False, True])
def test_append_identity_table_is_dense_write(oracle, packed):
    """With an identity block table the paged cache is a dense [B, MB*bs, G, D] cache, and the
    append must place new row t of sequence b at position past_b + t and touch nothing else."""
    w = _identity_table(_small(1, packed=packed))
    kc, vc = oracle.kv_append(w)
    B, MB, bs, G, D, H = w["B"], w["MB"], w["bs"], w["G"], w["D"], w["H"]
    dk = w["key_cache"].reshape(B, MB * bs, G, D).copy()
    dv = w["value_cache"].reshape(B, MB * bs, G, D).copy()
    for b in range(B):
        rows = slice(w["cu"][b], w["cu"][b + 1])
        n = w["cu"][b + 1] - w["cu"][b]
        if packed:
            k = w["query"][rows, H * D:(H + G) * D]
            v = w["query"][rows, (H + G) * D:]
        else:
            k, v = w["key"][rows], w["value"][rows]
        dk[b, w["past"][b]:w["past"][b] + n] = k.reshape(n, G, D)
        dv[b, w["past"][b]:w["past"][b] + n] = v.reshape(n, G, D)
    assert np.array_equal(kc.reshape(B, MB * bs, G, D).view(np.uint16), dk.view(np.uint16))
    assert np.array_equal(vc.reshape(B, MB * bs, G, D).view(np.uint16), dv.view(np.uint16))


def test_append_commutes_with_block_permutation(oracle):
    """Relabelling physical blocks (and the table with them) relabels the result the same way."""
    w = _small(2)
    kc, vc = oracle.kv_append(w)
    perm = np.random.default_rng(5).permutation(w["NB"])
    inv = np.argsort(perm)
    w2 = dict(w)
    w2["key_cache"] = w["key_cache"][perm]          # new block j holds old block perm[j]
    w2["value_cache"] = w["value_cache"][perm]
    bt = w["block_table"].copy()
    bt[bt >= 0] = inv[bt[bt >= 0]]
    w2["block_table"] = bt
    kc2, vc2 = oracle.kv_append(w2)
    assert np.array_equal(kc2.view(np.uint16), kc[perm].view(np.uint16))
    assert np.array_equal(vc2.view(np.uint16), vc[perm].view(np.uint16))


def test_append_writes_exactly_new_rows(oracle):
    """Only T*G key rows and T*G value rows change; every other cache byte is untouched."""
    w = _small(3)
    kc, vc = oracle.kv_append(w)
    rows_k = (kc.view(np.uint16) != w["key_cache"].view(np.uint16)).any(axis=-1)
    rows_v = (vc.view(np.uint16) != w["value_cache"].view(np.uint16)).any(axis=-1)
    assert rows_k.sum() == w["T"] * w["G"]
    assert rows_v.sum() == w["T"] * w["G"]


def test_slot_mapping_equals_derived_slots(oracle):
    w = _small(4, use_slot_mapping=True)
    a = oracle.kv_append(w)
    w2 = dict(w)
    w2["slot_mapping"] = None
    b = oracle.kv_append(w2)
    assert np.array_equal(a[0].view(np.uint16), b[0].view(np.uint16))
    assert np.array_equal(a[1].view(np.uint16), b[1].view(np.uint16))


def test_negative_slot_writes_nothing(oracle):
    w = _small(5, use_slot_mapping=True)
    w["slot_mapping"] = w["slot_mapping"].copy()
    w["slot_mapping"][:] = -1
    kc, vc = oracle.kv_append(w)
    assert np.array_equal(kc.view(np.uint16), w["key_cache"].view(np.uint16))
    assert np.array_equal(vc.view(np.uint16), w["value_cache"].view(np.uint16))


# ------------------------------------------------------------------ rotary
def _rot_workload(seed, mode, D=64, R=None, past=(0, 9, 40), n_new=(2, 3, 1), positions=64):
    R = D if R is None else R
    return W.paged_workload(seed, past=list(past), n_new=list(n_new), num_heads=2, kv_num_heads=2,
                            head_size=D, block_size=8, table="pool", slack=0.2,
                            rotary_mode=mode, rotary_dim=R, rotary_positions=positions,
                            name="rot")


def _new_key_rows(w, kc):
    """Read back new row t of each sequence through the workload's block table."""
    out = []
    for b in range(w["B"]):
        for t in range(w["cu"][b + 1] - w["cu"][b]):
            pos = w["past"][b] + t
            out.append(kc[w["block_table"][b, pos // w["bs"]], pos % w["bs"]])
    return np.stack(out)          # [T, G, D]


def _positions(w):
    return np.concatenate([w["past"][b] + np.arange(w["cu"][b + 1] - w["cu"][b])
                           for b in range(w["B"])])


@pytest.mark.parametrize("mode", [W.ROTARY_NEOX, W.ROTARY_INTERLEAVED])
def test_rotary_position_zero_is_identity(oracle, mode):
    """cos(0) = 1 and sin(0) = 0 are exact in fp16, so position 0 copies the key bit for bit."""
    w = _rot_workload(10, mode, past=(0,), n_new=(1,))
    kc, _ = oracle.kv_append(w)
    got = _new_key_rows(w, kc)
    assert np.array_equal(got.reshape(1, -1).view(np.uint16), w["key"].view(np.uint16))


def _complex_rotation_reference(w):
    """Rotary as complex multiplication, in float64: the pair (x_a, x_b) is z = x_a + i x_b and is
    multiplied by cos + i sin taken from the same fp16 tables. NeoX pairs (d, d+R/2); interleaved
    pairs (2i, 2i+1)."""
    R, D, G = w["rotary_dim"], w["D"], w["G"]
    half = R // 2
    k = w["key"].astype(np.float64).reshape(-1, G, D)
    pos = _positions(w)
    c = w["cos"].astype(np.float64)[pos][:, None, :]
    s = w["sin"].astype(np.float64)[pos][:, None, :]
    if w["rotary_mode"] == W.ROTARY_NEOX:
        a, bb = k[..., :half], k[..., half:R]
    else:
        a, bb = k[..., 0:R:2], k[..., 1:R:2]
    z = (a + 1j * bb) * (c + 1j * s)
    out = k.copy()
    if w["rotary_mode"] == W.ROTARY_NEOX:
        out[..., :half], out[..., half:R] = z.real, z.imag
    else:
        out[..., 0:R:2], out[..., 1:R:2] = z.real, z.imag
    return out


@pytest.mark.parametrize("mode", [W.ROTARY_NEOX, W.ROTARY_INTERLEAVED])
@pytest.mark.parametrize("D,R", [(64, 64), (128, 128), (64, 32)])
def test_rotary_matches_complex_multiplication(oracle, mode, D, R):
    """float32 rotary then fp16 rounding stays within half an fp16 ulp of the exact rotation plus
    the float32 rounding of two products and one sum (<= 2 float32 ulps of the operands)."""
    w = _rot_workload(11, mode, D=D, R=R)
    kc, _ = oracle.kv_append(w)
    got = _new_key_rows(w, kc).astype(np.float64)
    ref = _complex_rotation_reference(w)
    k = w["key"].astype(np.float64).reshape(ref.shape)
    half_ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64) / 2
    f32 = 4 * np.finfo(np.float32).eps * (np.abs(ref) + np.abs(k).max(axis=-1, keepdims=True))
    assert np.all(np.abs(got - ref) <= half_ulp + f32)
    # components past the rotary dimension are copied unchanged
    assert np.array_equal(got[..., R:], k[..., R:])


def _permute_interleaved_to_neox(x, R):
    """P: even components first, then odd ones (on the first R components)."""
    y = x.copy()
    y[..., :R // 2] = x[..., 0:R:2]
    y[..., R // 2:R] = x[..., 1:R:2]
    return y


def test_rotary_layouts_are_a_permutation_of_each_other(oracle):
    """interleaved(x) = P^-1 neox(P x) exactly: both apply the same per-pair arithmetic."""
    wi = _rot_workload(12, W.ROTARY_INTERLEAVED, D=128, R=128)
    wn = dict(wi)
    wn["rotary_mode"] = W.ROTARY_NEOX
    G, D, R = wi["G"], wi["D"], wi["rotary_dim"]
    kx = wi["key"].reshape(-1, G, D)
    wn["key"] = _permute_interleaved_to_neox(kx, R).reshape(wi["key"].shape)
    ki, _ = oracle.kv_append(wi)
    kn, _ = oracle.kv_append(wn)
    gi = _new_key_rows(wi, ki)
    gn = _new_key_rows(wn, kn)
    assert np.array_equal(_permute_interleaved_to_neox(gi, R).view(np.uint16), gn.view(np.uint16))


def test_rotary_quarter_turn_and_half_turn_exact(oracle):
    """With cos = 0, sin = 1 the pair (a, b) becomes (-b, a); with cos = -1, sin = 0 it becomes
    (-a, -b). Both are exact in fp16, so the result is bit-exact."""
    w = _rot_workload(13, W.ROTARY_NEOX, D=64, past=(1, 2), n_new=(1, 1), positions=4)
    half = 32
    cos = np.ones((4, half), np.float16)
    sin = np.zeros((4, half), np.float16)
    cos[1], sin[1] = 0.0, 1.0
    cos[2], sin[2] = -1.0, 0.0
    w["cos"], w["sin"] = cos, sin
    kc, _ = oracle.kv_append(w)
    got = _new_key_rows(w, kc)
    k = w["key"].reshape(2, w["G"], 64)
    q1 = np.concatenate([-k[0, :, half:], k[0, :, :half]], axis=-1)
    q2 = -k[1]
    assert np.array_equal(got[0].view(np.uint16), q1.view(np.uint16))
    assert np.array_equal(got[1].view(np.uint16), q2.view(np.uint16))


def test_rotary_preserves_pair_norm(oracle):
    w = _rot_workload(14, W.ROTARY_NEOX, D=128, R=128, positions=64)
    kc, _ = oracle.kv_append(w)
    got = _new_key_rows(w, kc).astype(np.float64)
    k = w["key"].astype(np.float64).reshape(got.shape)
    pos = _positions(w)
    c = w["cos"].astype(np.float64)[pos][:, None, :]
    s = w["sin"].astype(np.float64)[pos][:, None, :]
    n_in = np.hypot(k[..., :64], k[..., 64:]) * np.sqrt(c * c + s * s)
    n_out = np.hypot(got[..., :64], got[..., 64:])
    # each output component carries at most half an fp16 ulp (<= 2^-11 relative) of rounding
    assert np.all(np.abs(n_out - n_in) <= 2.0 ** -10 * n_in + 1e-6)
    # the fp16 tables themselves keep cos^2 + sin^2 within 2 fp16 ulps of 1
    assert np.all(np.abs(c * c + s * s - 1.0) < 2e-3)


# ------------------------------------------------------------------ query rotation
def _query_rows(w):
    """[T, H, D] float64 view of the new query rows (Q part of packed rows, or separate Q)."""
    T, H, G, D = w["T"], w["H"], w["G"], w["D"]
    q = w["query"].reshape(T, -1)[:, :H * D]
    return q.astype(np.float64).reshape(T, H, D)


@pytest.mark.parametrize("mode", [W.ROTARY_NEOX, W.ROTARY_INTERLEAVED])
@pytest.mark.parametrize("packed", [False, True])
def test_query_rotary_position_zero_is_identity(oracle, mode, packed):
    """cos(0) = 1, sin(0) = 0: position 0 copies every query head row bit for bit."""
    w = W.paged_workload(20, past=[0], n_new=[1], num_heads=4, kv_num_heads=2, head_size=64,
                         block_size=8, table="pool", packed=packed, rotary_mode=mode,
                         rotary_dim=64, rotary_positions=8, name="qrot0")
    got = oracle.rotate_query(w)
    H, D = w["H"], w["D"]
    src = w["query"].reshape(1, -1)[:, :H * D]
    assert np.array_equal(got.view(np.uint16), np.ascontiguousarray(src).view(np.uint16))


@pytest.mark.parametrize("mode", [W.ROTARY_NEOX, W.ROTARY_INTERLEAVED])
@pytest.mark.parametrize("D,R,packed", [(64, 64, False), (128, 128, True), (64, 32, False),
                                        (128, 48, True)])
def test_query_rotary_matches_complex_multiplication(oracle, mode, D, R, packed):
    """Each query head row rotated as complex multiplication in float64 (pairs as for keys), within
    half an fp16 ulp plus the float32 rounding of the page's expression; dims past R copied."""
    w = W.paged_workload(21, past=[0, 9, 40], n_new=[2, 3, 1], num_heads=6, kv_num_heads=2,
                         head_size=D, block_size=8, table="pool", packed=packed,
                         rotary_mode=mode, rotary_dim=R, rotary_positions=64, name="qrot")
    got = oracle.rotate_query(w).astype(np.float64).reshape(w["T"], w["H"], D)
    q = _query_rows(w)
    half = R // 2
    pos = _positions(w)
    c = w["cos"].astype(np.float64)[pos][:, None, :]
    s = w["sin"].astype(np.float64)[pos][:, None, :]
    if mode == W.ROTARY_NEOX:
        a, bb = q[..., :half], q[..., half:R]
    else:
        a, bb = q[..., 0:R:2], q[..., 1:R:2]
    z = (a + 1j * bb) * (c + 1j * s)
    ref = q.copy()
    if mode == W.ROTARY_NEOX:
        ref[..., :half], ref[..., half:R] = z.real, z.imag
    else:
        ref[..., 0:R:2], ref[..., 1:R:2] = z.real, z.imag
    half_ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64) / 2
    f32 = 4 * np.finfo(np.float32).eps * (np.abs(ref) + np.abs(q).max(axis=-1, keepdims=True))
    assert np.all(np.abs(got - ref) <= half_ulp + f32)
    assert np.array_equal(got[..., R:], q[..., R:])


@pytest.mark.parametrize("mode", [W.ROTARY_NEOX, W.ROTARY_INTERLEAVED])
def test_query_rotation_equals_key_rotation(oracle, mode):
    """With one query head per kv head, feeding the query rows in as keys makes the key path
    write exactly the rotated query rows into the cache."""
    w = _rot_workload(22, mode, D=128, R=128)
    wk = dict(w)
    wk["key"] = w["query"].reshape(w["key"].shape).copy()
    kc, _ = oracle.kv_append(wk)
    rows = _new_key_rows(wk, kc).reshape(w["T"], -1)
    assert np.array_equal(oracle.rotate_query(w).view(np.uint16), rows.view(np.uint16))


def test_query_rotation_none_copies(oracle):
    w = W.paged_workload(23, past=[3, 7], n_new=[2, 1], num_heads=4, kv_num_heads=1,
                         head_size=64, block_size=8, table="pool", packed=True, name="qcopy")
    got = oracle.rotate_query(w)
    src = np.ascontiguousarray(w["query"].reshape(w["T"], -1)[:, :4 * 64])
    assert np.array_equal(got.view(np.uint16), src.view(np.uint16))


# ------------------------------------------------------------------ contiguous BNSH append
def _bnsh(seed, **kw):
    args = dict(batch=3, seq_len=5, num_heads=4, kv_num_heads=2, head_size=64, max_seq=24,
                key_total=[9, 5, 21], name="bnsh_small")
    args.update(kw)
    return W.bnsh_workload(seed, **args)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("mode", [W.ROTARY_NONE, W.ROTARY_NEOX, W.ROTARY_INTERLEAVED])
def test_bnsh_equals_paged_append_with_one_block_per_sequence(oracle, packed, mode):
    """A BNSH cache [B, KVH, S_max, D] is a paged cache [B, S_max, KVH, D] (one block of S_max
    keys per sequence, identity table) with the two middle axes swapped. Feeding the padded rows
    to the (separately pinned) paged append with past = the padded-batch rule must give the same
    cache bits."""
    bw = _bnsh(40, packed=packed, rotary_mode=mode,
               rotary_dim=None if mode == W.ROTARY_NONE else 64)
    pk, pv = oracle.kv_append_bnsh(bw)
    B, S, KVH, D, M = bw["B"], bw["S"], bw["KVH"], bw["D"], bw["max_seq"]
    past = np.array([oracle.past_length_padded(bw["total_seq"], int(k), S)
                     for k in bw["key_total"]], dtype=np.int32)
    w = dict(T=B * S, B=B, H=bw["H"], G=KVH, D=D, bs=M, MB=1, NB=B, packed=packed,
             query=bw["query"], key=bw["key"], value=bw["value"],
             key_cache=np.ascontiguousarray(bw["present_key"].transpose(0, 2, 1, 3)),
             value_cache=np.ascontiguousarray(bw["present_value"].transpose(0, 2, 1, 3)),
             cu=np.arange(B + 1, dtype=np.int32) * S, past=past,
             block_table=np.arange(B, dtype=np.int32).reshape(B, 1), slot_mapping=None,
             cos=bw["cos"], sin=bw["sin"], rotary_dim=bw["rotary_dim"],
             rotary_mode=bw["rotary_mode"])
    kc, vc = oracle.kv_append(w)
    assert np.array_equal(pk.view(np.uint16), kc.transpose(0, 2, 1, 3).view(np.uint16))
    assert np.array_equal(pv.view(np.uint16), vc.transpose(0, 2, 1, 3).view(np.uint16))


def test_bnsh_prompt_mode_writes_from_position_zero(oracle):
    """Scalar total == seq_len: every row (even one whose own total is larger) starts at 0."""
    bw = _bnsh(41, key_total=[5, 12, 3], total_seq=5)
    pk, _ = oracle.kv_append_bnsh(bw)
    B, S, KVH, D = bw["B"], bw["S"], bw["KVH"], bw["D"]
    k = bw["key"].reshape(B, S, KVH, D).transpose(0, 2, 1, 3)
    assert np.array_equal(pk[:, :, :S].view(np.uint16), k.view(np.uint16))
    assert np.array_equal(pk[:, :, S:].view(np.uint16), bw["present_key"][:, :, S:].view(np.uint16))


def test_bnsh_rows_past_the_cache_are_not_written(oracle):
    bw = _bnsh(42, key_total=[26, 5, 21])       # batch 0: past 21, rows 21..25, cache holds 24
    pk, pv = oracle.kv_append_bnsh(bw)
    k = bw["key"].reshape(3, 5, 2, 64).transpose(0, 2, 1, 3)
    assert np.array_equal(pk[0, :, 21:24].view(np.uint16), k[0, :, :3].view(np.uint16))
    changed = pk.view(np.uint16) != bw["present_key"].view(np.uint16)
    assert changed[0, :, 21:24].any() and not changed[0, :, :21].any()
    assert not changed[1, :, 5:].any() and not changed[2, :, :16].any()
