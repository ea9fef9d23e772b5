"""Host-only checks of the C ABI: the library loads, exports every function include/pa.h
declares, and rejects contract violations (the PagedAttention manifest's cacheShapeOk,
headLayoutOk, scheduleShapeOk, separateKv/packedKv and is_causal rules; the sparse page's
Params) before it enqueues anything. No call here reaches a GPU: every argument set fails
validation, or is empty, or only sizes a workspace."""
import os
import re

import pytest

import block_sparse_gqa_paged_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20   # a non-NULL address that validation never dereferences


def _declared():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = pa.lib()
    declared = _declared()
    assert set(declared) == set(pa.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def _shape(**kw):
    a = dict(batch=2, num_tokens=2, num_heads=4, kv_num_heads=2, head_size=64, num_blocks=16,
             block_size=16, max_blocks=8, packed_qkv=False)
    a.update(kw)
    return pa.paged_shape(**a)


def _append(shape, **kw):
    a = dict(query=None, key=FAKE, value=FAKE, key_cache=FAKE, value_cache=FAKE,
             cumulative_sequence_length=FAKE, past_seqlens=FAKE, block_table=FAKE,
             slot_mapping=None, cos_cache=None, sin_cache=None, rotary_dim=0,
             rotary_mode=pa.PA_ROTARY_NONE, rotary_positions=0, stream=0, check=False)
    a.update(kw)
    return pa.pa_kv_append(shape, **a)


@pytest.mark.parametrize("bad,expect", [
    (dict(batch=0), pa.PA_ERR_SHAPE),
    (dict(num_heads=6, kv_num_heads=4), pa.PA_ERR_SHAPE),      # H % G != 0
    (dict(kv_num_heads=0), pa.PA_ERR_SHAPE),
    (dict(block_size=0), pa.PA_ERR_SHAPE),
    (dict(max_blocks=0), pa.PA_ERR_SHAPE),
    (dict(num_blocks=0), pa.PA_ERR_SHAPE),
    (dict(num_tokens=-1), pa.PA_ERR_SHAPE),
    (dict(head_size=96), pa.PA_ERR_UNSUPPORTED),
    (dict(head_size=512), pa.PA_ERR_UNSUPPORTED),
    # a block's elements must fit in 32 bits (24-bit in-block offset products)
    (dict(num_heads=64, kv_num_heads=64, head_size=128, block_size=1 << 19),
     pa.PA_ERR_UNSUPPORTED),
])
def test_append_rejects_bad_shapes(bad, expect):
    assert _append(_shape(**bad)) == expect


def test_append_kv_presence_rules():
    # separate layout needs both key and value; packed needs neither
    assert _append(_shape(), value=None) == pa.PA_ERR_SHAPE
    assert _append(_shape(), key=None, value=None) == pa.PA_ERR_NULL
    assert _append(_shape(packed_qkv=True), query=FAKE) == pa.PA_ERR_SHAPE
    assert _append(_shape(packed_qkv=True), query=None, key=None, value=None) == pa.PA_ERR_NULL
    assert _append(_shape(), key_cache=None) == pa.PA_ERR_NULL
    assert _append(_shape(), block_table=None) == pa.PA_ERR_NULL  # no slots without either


def test_append_rotary_rules():
    rot = dict(cos_cache=FAKE, sin_cache=FAKE, rotary_mode=pa.PA_ROTARY_NEOX,
               rotary_positions=4)
    assert _append(_shape(), rotary_dim=63, **rot) == pa.PA_ERR_SHAPE
    assert _append(_shape(), rotary_dim=128, **rot) == pa.PA_ERR_SHAPE
    assert _append(_shape(), rotary_dim=0, **rot) == pa.PA_ERR_SHAPE
    assert _append(_shape(), rotary_dim=64, rotary_mode=3, rotary_positions=4) == pa.PA_ERR_SHAPE
    rot["cos_cache"] = None
    assert _append(_shape(), rotary_dim=64, **rot) == pa.PA_ERR_NULL


def test_rotate_query_rules():
    def rq(shape, **kw):
        a = dict(query=FAKE, key=FAKE, value=FAKE, key_cache=FAKE, value_cache=FAKE,
                 cumulative_sequence_length=FAKE, past_seqlens=FAKE, block_table=FAKE,
                 q_out=FAKE + 4096, stream=0, check=False)
        a.update(kw)
        return pa.pa_kv_append_rotate_query(shape, **a)
    assert rq(_shape(), q_out=None) == pa.PA_ERR_NULL
    assert rq(_shape(), query=None) == pa.PA_ERR_NULL
    assert rq(_shape(), q_out=FAKE) == pa.PA_ERR_SHAPE             # rotated rows need own buffer
    assert rq(_shape(batch=0)) == pa.PA_ERR_SHAPE
    assert rq(_shape(), value=None) == pa.PA_ERR_SHAPE            # the append's own rules hold
    assert rq(_shape(num_tokens=0)) == pa.PA_OK


def test_empty_append_is_a_no_op():
    assert _append(_shape(num_tokens=0)) == pa.PA_OK


def _attn(shape, **kw):
    a = dict(query=FAKE, key_cache=FAKE, value_cache=FAKE, cumulative_sequence_length=FAKE,
             past_seqlens=FAKE, block_table=FAKE, scale=0.0, causal=1,
             num_splits=pa.PA_SPLITS_AUTO, workspace=FAKE, workspace_bytes=0, output=FAKE,
             stream=0, check=False)
    a.update(kw)
    return pa.pa_paged_attention(shape, **a)


def test_attention_rejects_bad_arguments():
    assert _attn(_shape(), causal=2) == pa.PA_ERR_SHAPE          # is_causal values [1] (+0)
    assert _attn(_shape(), num_splits=-2) == pa.PA_ERR_SHAPE
    assert _attn(_shape(), block_table=None) == pa.PA_ERR_NULL
    assert _attn(_shape(), output=None) == pa.PA_ERR_NULL
    assert _attn(_shape(head_size=512)) == pa.PA_ERR_UNSUPPORTED
    assert _attn(_shape(), workspace_bytes=16) == pa.PA_ERR_WORKSPACE
    n = pa.pa_paged_attention_workspace_size(_shape())
    assert _attn(_shape(), workspace=FAKE + 4, workspace_bytes=n) == pa.PA_ERR_WORKSPACE
    assert _attn(_shape(num_tokens=0), workspace=None) == pa.PA_OK


def _append_attn(shape, **kw):
    a = dict(query=FAKE, key=FAKE, value=FAKE, key_cache=FAKE, value_cache=FAKE,
             cumulative_sequence_length=FAKE, past_seqlens=FAKE, block_table=FAKE, scale=0.0,
             causal=1, num_splits=pa.PA_SPLITS_AUTO, workspace=FAKE,
             workspace_bytes=pa.pa_paged_attention_workspace_size(shape), output=FAKE,
             stream=0, check=False)
    a.update(kw)
    return pa.pa_append_attention(shape, **a)


def test_append_attention_checks_both_parts_before_enqueueing():
    # Each argument set breaks one rule of the append or of the attention; the call must report
    # it before enqueueing anything (a launch here, without a GPU, would report PA_ERR_HIP).
    assert _append_attn(_shape(), query=None) == pa.PA_ERR_NULL
    assert _append_attn(_shape(), q_out=FAKE) == pa.PA_ERR_SHAPE        # q_out == query
    assert _append_attn(_shape(), value=None) == pa.PA_ERR_SHAPE        # append: key xor value
    assert _append_attn(_shape(packed_qkv=True)) == pa.PA_ERR_SHAPE     # packed with key/value
    assert _append_attn(_shape(), key_cache=None) == pa.PA_ERR_NULL
    assert _append_attn(_shape(), rotary_dim=63, cos_cache=FAKE, sin_cache=FAKE,
                        rotary_mode=pa.PA_ROTARY_NEOX, rotary_positions=4) == pa.PA_ERR_SHAPE
    assert _append_attn(_shape(), causal=2) == pa.PA_ERR_SHAPE         # attention rules
    assert _append_attn(_shape(), num_splits=-2) == pa.PA_ERR_SHAPE
    assert _append_attn(_shape(), block_table=None) == pa.PA_ERR_NULL
    assert _append_attn(_shape(), output=None) == pa.PA_ERR_NULL
    assert _append_attn(_shape(), workspace_bytes=16) == pa.PA_ERR_WORKSPACE
    assert _append_attn(_shape(), workspace=FAKE + 4) == pa.PA_ERR_WORKSPACE
    assert _append_attn(_shape(), workspace=None) == pa.PA_ERR_NULL
    assert _append_attn(_shape(head_size=96)) == pa.PA_ERR_UNSUPPORTED
    assert _append_attn(_shape(batch=0)) == pa.PA_ERR_SHAPE
    assert _append_attn(_shape(num_tokens=0), workspace=None) == pa.PA_OK


def test_noalloc_rejects_before_any_hip_call():
    """pa_paged_attention_noalloc checks its shape against the static array's size before it
    makes any HIP call: a split count whose partials need more than PA_NOALLOC_SCRATCH_BYTES is
    PA_ERR_WORKSPACE, and the other argument errors are those of pa_paged_attention."""
    def na(shape, **kw):
        a = dict(query=FAKE, key_cache=FAKE, value_cache=FAKE, cumulative_sequence_length=FAKE,
                 past_seqlens=FAKE, block_table=FAKE, scale=0.0, causal=1,
                 num_splits=pa.PA_SPLITS_AUTO, output=FAKE, stream=0, check=False)
        a.update(kw)
        return pa.pa_paged_attention_noalloc(shape, **a)
    big = _shape(batch=64, num_tokens=4096, num_heads=32, kv_num_heads=8, head_size=128,
                 num_blocks=100000, block_size=16, max_blocks=4096)
    assert pa.pa_paged_attention_workspace_size(big, 16) > pa.PA_NOALLOC_SCRATCH_BYTES
    assert na(big, num_splits=16) == pa.PA_ERR_WORKSPACE
    assert na(_shape(), causal=2) == pa.PA_ERR_SHAPE
    assert na(_shape(), num_splits=-2) == pa.PA_ERR_SHAPE
    assert na(_shape(head_size=96)) == pa.PA_ERR_UNSUPPORTED
    assert na(_shape(), block_table=None) == pa.PA_ERR_NULL
    assert na(_shape(), output=None) == pa.PA_ERR_NULL
    assert na(_shape(num_tokens=0)) == pa.PA_OK


def test_workspace_size_is_zero_for_invalid_shapes():
    assert pa.pa_paged_attention_workspace_size(_shape(batch=0)) == 0
    assert pa.pa_paged_attention_workspace_size(_shape(), -3) == 0
    assert pa.pa_paged_attention_workspace_size(_shape()) > 0


@pytest.mark.parametrize("shape,expect_s", [
    # the manifest's numSplits: min(cap, ceil(1024 / (T*G))), cap = min(16, MB*bs/128)
    (dict(batch=2, num_tokens=2, num_heads=4, kv_num_heads=2, head_size=64, block_size=16,
          max_blocks=8), 1),                                        # tiny decode: cap 1
    (dict(batch=4, num_tokens=4, num_heads=8, kv_num_heads=8, head_size=128, block_size=32,
          max_blocks=128), 16),                                     # rotary decode
    (dict(batch=64, num_tokens=64, num_heads=32, kv_num_heads=8, head_size=128, block_size=16,
          max_blocks=513), 2),                                      # GQA serving decode
    (dict(batch=64, num_tokens=4152, num_heads=32, kv_num_heads=8, head_size=128,
          block_size=32, max_blocks=513), 1),                       # mixed prefill + decode
])
def test_page_rule_split_count(shape, expect_s):
    s = _shape(**shape)
    assert (pa.pa_paged_attention_workspace_size(s, pa.PA_SPLITS_PAGE_RULE) ==
            pa.pa_paged_attention_workspace_size(s, expect_s))
    if expect_s > 1:
        assert (pa.pa_paged_attention_workspace_size(s, expect_s) >
                pa.pa_paged_attention_workspace_size(s, 1))


def test_combine_rejects_bad_arguments():
    def comb(**kw):
        a = dict(o_partial=FAKE, m_partial=FAKE, l_partial=FAKE, group_ptr=None, num_groups=4,
                 lanes=4, num_splits=2, head_dim=128, out_dtype=pa.PA_F32, out=FAKE, stream=0,
                 check=False)
        a.update(kw)
        return pa.pa_split_combine(**a)
    assert comb(lanes=0) == pa.PA_ERR_SHAPE
    assert comb(num_groups=-1) == pa.PA_ERR_SHAPE
    assert comb(num_splits=0) == pa.PA_ERR_SHAPE
    assert comb(out_dtype=7) == pa.PA_ERR_SHAPE
    assert comb(head_dim=30) == pa.PA_ERR_SHAPE
    assert comb(head_dim=96) == pa.PA_ERR_UNSUPPORTED
    assert comb(out=None) == pa.PA_ERR_NULL
    assert comb(num_groups=0, out=None) == pa.PA_OK


def test_sparse_rejects_bad_arguments():
    def sh(**kw):
        a = dict(num_edges=10, tq=8, hkv=2, qhead=4, head_dim=128, block_size=64, page_size=16,
                 num_pages=64, max_pages=32, batch=2)
        a.update(kw)
        return pa.sparse_shape(**a)

    def fwd(shape, **kw):
        a = dict(q_buf=FAKE, k_pages=FAKE, v_pages=FAKE, edge_meta=FAKE, block_tables=FAKE,
                 softmax_scale=0.1, causal=0, workspace=FAKE, workspace_bytes=0, o_partial=FAKE,
                 m_partial=FAKE, l_partial=FAKE, stream=0, check=False)
        a.update(kw)
        return pa.pa_sparse_forward(shape, **a)
    assert fwd(sh(), causal=1) == pa.PA_ERR_UNSUPPORTED     # right-aligned causal unimplemented
    assert fwd(sh(block_size=60)) == pa.PA_ERR_SHAPE          # not a multiple of page_size
    assert fwd(sh(block_size=256)) == pa.PA_ERR_UNSUPPORTED
    assert fwd(sh(head_dim=256, block_size=128)) == pa.PA_ERR_UNSUPPORTED  # planes beyond LDS
    assert fwd(sh(qhead=32), workspace_bytes=8) == pa.PA_ERR_WORKSPACE   # any qhead: checked on
    assert fwd(sh(head_dim=80)) == pa.PA_ERR_UNSUPPORTED
    assert fwd(sh(), edge_meta=None) == pa.PA_ERR_NULL
    assert fwd(sh(), workspace_bytes=8) == pa.PA_ERR_WORKSPACE
    assert fwd(sh(num_edges=0), q_buf=None) == pa.PA_OK

    def cfwd(shape, **kw):
        a = dict(q_buf=FAKE, k_pages=FAKE, v_pages=FAKE, edge_meta=FAKE, block_tables=FAKE,
                 q_pos=FAKE, softmax_scale=0.1, workspace=FAKE, workspace_bytes=0,
                 o_partial=FAKE, m_partial=FAKE, l_partial=FAKE, stream=0, check=False)
        a.update(kw)
        return pa.pa_sparse_forward_causal(shape, **a)
    assert cfwd(sh(), q_pos=None) == pa.PA_ERR_NULL            # the mask needs positions
    assert cfwd(sh(block_size=60)) == pa.PA_ERR_SHAPE
    assert cfwd(sh(), workspace_bytes=8) == pa.PA_ERR_WORKSPACE
    assert cfwd(sh(num_edges=0), q_pos=None) == pa.PA_OK
    assert pa.pa_sparse_forward_workspace_size(sh()) > 0
    assert pa.pa_sparse_forward_workspace_size(sh(hkv=0)) == 0


def test_status_strings():
    for s in range(6):
        assert pa.status_string(s)
    assert "unknown" in pa.status_string(99)


def test_build_edges_rejects_bad_arguments():
    def be(**kw):
        a = dict(tq=4, hkv=2, nblk=8, block_size=16, batch=1, block_mask=FAKE, q_batch=FAKE,
                 used_kv_lens=FAKE, edge_capacity=64, edge_meta=FAKE, group_ptr=FAKE,
                 workspace=FAKE, workspace_bytes=1 << 20, stream=0, check=False)
        a.update(kw)
        return pa.pa_sparse_build_edges(**a)
    assert be(tq=-1) == pa.PA_ERR_SHAPE
    assert be(hkv=0) == pa.PA_ERR_SHAPE
    assert be(nblk=0) == pa.PA_ERR_SHAPE
    assert be(edge_capacity=-1) == pa.PA_ERR_SHAPE
    assert be(tq=1 << 20, hkv=64, nblk=64) == pa.PA_ERR_UNSUPPORTED   # >= 2^31 mask entries
    assert be(group_ptr=None) == pa.PA_ERR_NULL
    assert be(block_mask=None) == pa.PA_ERR_NULL
    assert be(edge_meta=None) == pa.PA_ERR_NULL
    assert be(workspace_bytes=4) == pa.PA_ERR_WORKSPACE
    assert be(workspace=FAKE + 4) == pa.PA_ERR_WORKSPACE
    assert pa.pa_sparse_build_edges_workspace_size(4, 2) >= 256
    assert pa.pa_sparse_build_edges_workspace_size(-1, 2) == 0


def test_bnsh_append_rejects_bad_arguments():
    def sh(**kw):
        a = dict(batch=2, seq_len=4, num_heads=4, kv_num_heads=2, head_size=64, max_cache_seq=32,
                 packed_qkv=False)
        a.update(kw)
        return pa.bnsh_shape(**a)

    def ap(shape, **kw):
        a = dict(query=None, key=FAKE, value=FAKE, present_key=FAKE, present_value=FAKE,
                 total_sequence_length=FAKE, key_total_sequence_lengths=FAKE, stream=0,
                 check=False)
        a.update(kw)
        return pa.pa_kv_append_bnsh(shape, **a)
    assert ap(sh(batch=0)) == pa.PA_ERR_SHAPE
    assert ap(sh(num_heads=6, kv_num_heads=4)) == pa.PA_ERR_SHAPE
    assert ap(sh(max_cache_seq=0)) == pa.PA_ERR_SHAPE
    assert ap(sh(head_size=96)) == pa.PA_ERR_UNSUPPORTED
    assert ap(sh(), value=None) == pa.PA_ERR_SHAPE
    assert ap(sh(packed_qkv=True)) == pa.PA_ERR_SHAPE                  # packed: no key/value
    assert ap(sh(packed_qkv=True), key=None, value=None) == pa.PA_ERR_NULL
    assert ap(sh(), rotary_mode=pa.PA_ROTARY_NEOX, rotary_dim=64, rotary_positions=8) == \
        pa.PA_ERR_NULL                                                # tables missing
    assert ap(sh(), rotary_mode=pa.PA_ROTARY_NEOX, rotary_dim=63, rotary_positions=8,
              cos_cache=FAKE, sin_cache=FAKE) == pa.PA_ERR_SHAPE
    assert ap(sh(), present_key=None) == pa.PA_ERR_NULL
    assert ap(sh(seq_len=0), present_key=None) == pa.PA_OK


def test_check_paged_indices_rejects_bad_arguments():
    f = lambda shape, **kw: pa.pa_check_paged_indices(
        shape, kw.get("cu", FAKE), kw.get("past", FAKE), FAKE, None, kw.get("flags", FAKE),
        rotary_positions=kw.get("rot", 0), stream=0, check=False)
    assert f(_shape(), flags=None) == pa.PA_ERR_NULL
    assert f(_shape(), cu=None) == pa.PA_ERR_NULL
    assert f(_shape(), past=None) == pa.PA_ERR_NULL
    assert f(_shape(batch=0)) == pa.PA_ERR_SHAPE
    assert f(_shape(head_size=96)) == pa.PA_ERR_UNSUPPORTED
    assert f(_shape(), rot=-1) == pa.PA_ERR_SHAPE
