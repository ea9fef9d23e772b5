"""Python binding of libpa, the MI355X (gfx950) paged GQA attention library.

The functions here have the names of the C entry points in include/pa.h and only marshal
arguments: tensors become device pointers (``tensor.data_ptr()``), ``stream=None`` becomes the
current torch stream, and a non-zero pa_status raises :class:`PAError`. Every step of the
computation runs in the HIP kernels of libpa.so; there is no CPU or PyTorch fallback, and
importing a missing library raises.

Build the library with ``python -m block_sparse_gqa_paged_amd._build`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(6)
PA_ROTARY_NONE, PA_ROTARY_NEOX, PA_ROTARY_INTERLEAVED = 0, 1, 2
PA_F16, PA_F32 = 0, 1
PA_SPLITS_AUTO, PA_SPLITS_PAGE_RULE = 0, -1
# pa_check_paged_indices flag bits (include/pa.h)
PA_CHECK_CU_START, PA_CHECK_CU_ORDER, PA_CHECK_CU_END, PA_CHECK_PAST = 1, 2, 4, 8
PA_CHECK_TABLE_WIDTH, PA_CHECK_TABLE_ENTRY, PA_CHECK_SLOT = 16, 32, 64
PA_CHECK_SLOT_TABLE, PA_CHECK_POSITION, PA_CHECK_SLOT_DUP = 128, 256, 512

EXPORTED = ("pa_kv_append", "pa_kv_append_rotate_query", "pa_paged_attention_workspace_size",
            "pa_paged_attention", "pa_paged_attention_noalloc", "pa_append_attention",
            "pa_split_combine", "pa_sparse_forward_workspace_size", "pa_sparse_forward",
            "pa_sparse_forward_causal", "pa_sparse_build_edges_workspace_size",
            "pa_sparse_build_edges", "pa_kv_append_bnsh", "pa_check_paged_indices",
            "pa_status_string", "pa_timing_enable", "pa_timing_reset", "pa_timing_get")


class PagedShape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_tokens", C.c_int32), ("num_heads", C.c_int32),
                ("kv_num_heads", C.c_int32), ("head_size", C.c_int32),
                ("num_blocks", C.c_int32), ("block_size", C.c_int32),
                ("max_blocks", C.c_int32), ("packed_qkv", C.c_int32)]


class SparseShape(C.Structure):
    _fields_ = [("num_edges", C.c_int32), ("tq", C.c_int32), ("hkv", C.c_int32),
                ("qhead", C.c_int32), ("head_dim", C.c_int32), ("block_size", C.c_int32),
                ("page_size", C.c_int32), ("num_pages", C.c_int32), ("max_pages", C.c_int32),
                ("batch", C.c_int32)]


class BnshShape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("seq_len", C.c_int32), ("num_heads", C.c_int32),
                ("kv_num_heads", C.c_int32), ("head_size", C.c_int32),
                ("max_cache_seq", C.c_int32), ("packed_qkv", C.c_int32)]


class PAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: pa_status {status} ({status_string(status)})")


_lib = None
_vp = C.c_void_p
_i32 = C.c_int32


def lib():
    """Load libpa.so (once). Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libpa.so not built at {LIB_PATH}; run "
                          "`python -m block_sparse_gqa_paged_amd._build`")
    L = C.CDLL(LIB_PATH)
    sp = C.POINTER(PagedShape)
    ss = C.POINTER(SparseShape)
    L.pa_kv_append.argtypes = [sp] + [_vp] * 11 + [_i32, _i32, _i32, _vp]
    L.pa_kv_append.restype = _i32
    L.pa_kv_append_rotate_query.argtypes = [sp] + [_vp] * 11 + [_i32, _i32, _i32, _vp, _vp]
    L.pa_kv_append_rotate_query.restype = _i32
    L.pa_paged_attention_workspace_size.argtypes = [sp, _i32]
    L.pa_paged_attention_workspace_size.restype = C.c_size_t
    L.pa_paged_attention.argtypes = ([sp] + [_vp] * 6 + [C.c_float, _i32, _i32, _vp, C.c_size_t,
                                                         _vp, _vp])
    L.pa_paged_attention.restype = _i32
    L.pa_paged_attention_noalloc.argtypes = [sp] + [_vp] * 6 + [C.c_float, _i32, _i32, _vp,
                                                                _vp]
    L.pa_paged_attention_noalloc.restype = _i32
    L.pa_append_attention.argtypes = ([sp] + [_vp] * 11 + [_i32, _i32, _i32, _vp, C.c_float,
                                      _i32, _i32, _vp, C.c_size_t, _vp, _vp])
    L.pa_append_attention.restype = _i32
    L.pa_split_combine.argtypes = [_vp] * 4 + [_i32] * 5 + [_vp, _vp]
    L.pa_split_combine.restype = _i32
    L.pa_sparse_forward_workspace_size.argtypes = [ss]
    L.pa_sparse_forward_workspace_size.restype = C.c_size_t
    L.pa_sparse_forward.argtypes = ([ss] + [_vp] * 5 + [C.c_float, _i32, _vp, C.c_size_t]
                                    + [_vp] * 4)
    L.pa_sparse_forward.restype = _i32
    L.pa_sparse_forward_causal.argtypes = ([ss] + [_vp] * 6 + [C.c_float, _vp, C.c_size_t]
                                           + [_vp] * 4)
    L.pa_sparse_forward_causal.restype = _i32
    L.pa_sparse_build_edges_workspace_size.argtypes = [_i32, _i32]
    L.pa_sparse_build_edges_workspace_size.restype = C.c_size_t
    L.pa_sparse_build_edges.argtypes = ([_i32] * 5 + [_vp] * 3 + [C.c_int64, _vp, _vp, _vp,
                                        C.c_size_t, _vp])
    L.pa_sparse_build_edges.restype = _i32
    L.pa_kv_append_bnsh.argtypes = [C.POINTER(BnshShape)] + [_vp] * 9 + [_i32] * 3 + [_vp]
    L.pa_kv_append_bnsh.restype = _i32
    L.pa_check_paged_indices.argtypes = [sp] + [_vp] * 4 + [_i32, _vp, _vp]
    L.pa_check_paged_indices.restype = _i32
    L.pa_status_string.argtypes = [_i32]
    L.pa_status_string.restype = C.c_char_p
    L.pa_timing_enable.argtypes = [_i32]
    L.pa_timing_enable.restype = None
    L.pa_timing_reset.argtypes = []
    L.pa_timing_reset.restype = None
    L.pa_timing_get.argtypes = [C.c_char_p, C.POINTER(C.c_double), C.POINTER(C.c_int64)]
    L.pa_timing_get.restype = _i32
    _lib = L
    return L


def _p(x):
    """Device pointer of a tensor (or an int address, or None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where, check):
    if check and status != PA_OK:
        raise PAError(status, where)
    return status


def status_string(status):
    return lib().pa_status_string(int(status)).decode()


def paged_shape(batch, num_tokens, num_heads, kv_num_heads, head_size, num_blocks, block_size,
                max_blocks, packed_qkv=False):
    return PagedShape(batch, num_tokens, num_heads, kv_num_heads, head_size, num_blocks,
                      block_size, max_blocks, int(bool(packed_qkv)))


def sparse_shape(num_edges, tq, hkv, qhead, head_dim, block_size, page_size, num_pages,
                 max_pages, batch):
    return SparseShape(num_edges, tq, hkv, qhead, head_dim, block_size, page_size, num_pages,
                       max_pages, batch)


# ------------------------------------------------------------------------------ entry points
def pa_kv_append(shape, query, key, value, key_cache, value_cache, cumulative_sequence_length,
                 past_seqlens, block_table, slot_mapping=None, cos_cache=None, sin_cache=None,
                 rotary_dim=0, rotary_mode=PA_ROTARY_NONE, rotary_positions=0, stream=None,
                 check=True):
    st = lib().pa_kv_append(
        C.byref(shape), _p(query), _p(key), _p(value), _p(key_cache), _p(value_cache),
        _p(cumulative_sequence_length), _p(past_seqlens), _p(block_table), _p(slot_mapping),
        _p(cos_cache), _p(sin_cache), int(rotary_dim), int(rotary_mode), int(rotary_positions),
        _s(stream))
    return _check(st, "pa_kv_append", check)


def pa_kv_append_rotate_query(shape, query, key, value, key_cache, value_cache,
                              cumulative_sequence_length, past_seqlens, block_table, q_out,
                              slot_mapping=None, cos_cache=None, sin_cache=None, rotary_dim=0,
                              rotary_mode=PA_ROTARY_NONE, rotary_positions=0, stream=None,
                              check=True):
    st = lib().pa_kv_append_rotate_query(
        C.byref(shape), _p(query), _p(key), _p(value), _p(key_cache), _p(value_cache),
        _p(cumulative_sequence_length), _p(past_seqlens), _p(block_table), _p(slot_mapping),
        _p(cos_cache), _p(sin_cache), int(rotary_dim), int(rotary_mode), int(rotary_positions),
        _p(q_out), _s(stream))
    return _check(st, "pa_kv_append_rotate_query", check)


def pa_paged_attention_workspace_size(shape, num_splits=PA_SPLITS_AUTO):
    return int(lib().pa_paged_attention_workspace_size(C.byref(shape), int(num_splits)))


def pa_paged_attention(shape, query, key_cache, value_cache, cumulative_sequence_length,
                       past_seqlens, block_table, scale, causal, num_splits, workspace,
                       workspace_bytes, output, stream=None, check=True):
    st = lib().pa_paged_attention(
        C.byref(shape), _p(query), _p(key_cache), _p(value_cache),
        _p(cumulative_sequence_length), _p(past_seqlens), _p(block_table), float(scale),
        int(causal), int(num_splits), _p(workspace), int(workspace_bytes), _p(output),
        _s(stream))
    return _check(st, "pa_paged_attention", check)


PA_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/pa.h


def pa_paged_attention_noalloc(shape, query, key_cache, value_cache, cumulative_sequence_length,
                               past_seqlens, block_table, scale, causal, num_splits, output,
                               stream=None, check=True):
    st = lib().pa_paged_attention_noalloc(
        C.byref(shape), _p(query), _p(key_cache), _p(value_cache),
        _p(cumulative_sequence_length), _p(past_seqlens), _p(block_table), float(scale),
        int(causal), int(num_splits), _p(output), _s(stream))
    return _check(st, "pa_paged_attention_noalloc", check)


def pa_append_attention(shape, query, key, value, key_cache, value_cache,
                        cumulative_sequence_length, past_seqlens, block_table, scale, causal,
                        num_splits, workspace, workspace_bytes, output, slot_mapping=None,
                        cos_cache=None, sin_cache=None, rotary_dim=0,
                        rotary_mode=PA_ROTARY_NONE, rotary_positions=0, q_out=None,
                        stream=None, check=True):
    st = lib().pa_append_attention(
        C.byref(shape), _p(query), _p(key), _p(value), _p(key_cache), _p(value_cache),
        _p(cumulative_sequence_length), _p(past_seqlens), _p(block_table), _p(slot_mapping),
        _p(cos_cache), _p(sin_cache), int(rotary_dim), int(rotary_mode), int(rotary_positions),
        _p(q_out), float(scale), int(causal), int(num_splits), _p(workspace),
        int(workspace_bytes), _p(output), _s(stream))
    return _check(st, "pa_append_attention", check)


def pa_split_combine(o_partial, m_partial, l_partial, group_ptr, num_groups, lanes, num_splits,
                     head_dim, out_dtype, out, stream=None, check=True):
    st = lib().pa_split_combine(_p(o_partial), _p(m_partial), _p(l_partial), _p(group_ptr),
                                int(num_groups), int(lanes), int(num_splits), int(head_dim),
                                int(out_dtype), _p(out), _s(stream))
    return _check(st, "pa_split_combine", check)


def pa_sparse_forward_workspace_size(shape):
    return int(lib().pa_sparse_forward_workspace_size(C.byref(shape)))


def pa_sparse_forward(shape, q_buf, k_pages, v_pages, edge_meta, block_tables, softmax_scale,
                      causal, workspace, workspace_bytes, o_partial, m_partial, l_partial,
                      stream=None, check=True):
    st = lib().pa_sparse_forward(
        C.byref(shape), _p(q_buf), _p(k_pages), _p(v_pages), _p(edge_meta), _p(block_tables),
        float(softmax_scale), int(causal), _p(workspace), int(workspace_bytes), _p(o_partial),
        _p(m_partial), _p(l_partial), _s(stream))
    return _check(st, "pa_sparse_forward", check)


def pa_sparse_forward_causal(shape, q_buf, k_pages, v_pages, edge_meta, block_tables, q_pos,
                             softmax_scale, workspace, workspace_bytes, o_partial, m_partial,
                             l_partial, stream=None, check=True):
    st = lib().pa_sparse_forward_causal(
        C.byref(shape), _p(q_buf), _p(k_pages), _p(v_pages), _p(edge_meta), _p(block_tables),
        _p(q_pos), float(softmax_scale), _p(workspace), int(workspace_bytes), _p(o_partial),
        _p(m_partial), _p(l_partial), _s(stream))
    return _check(st, "pa_sparse_forward_causal", check)


def pa_sparse_build_edges_workspace_size(tq, hkv):
    return int(lib().pa_sparse_build_edges_workspace_size(int(tq), int(hkv)))


def pa_sparse_build_edges(tq, hkv, nblk, block_size, batch, block_mask, q_batch, used_kv_lens,
                          edge_capacity, edge_meta, group_ptr, workspace, workspace_bytes,
                          stream=None, check=True):
    st = lib().pa_sparse_build_edges(
        int(tq), int(hkv), int(nblk), int(block_size), int(batch), _p(block_mask), _p(q_batch),
        _p(used_kv_lens), int(edge_capacity), _p(edge_meta), _p(group_ptr), _p(workspace),
        int(workspace_bytes), _s(stream))
    return _check(st, "pa_sparse_build_edges", check)


def pa_check_paged_indices(shape, cumulative_sequence_length, past_seqlens, block_table,
                           slot_mapping, flags, rotary_positions=0, stream=None, check=True):
    """Enqueue the device check of a paged call's index arrays; flags (int32 [1], device) gets
    one PA_CHECK_* bit per violated rule."""
    st = lib().pa_check_paged_indices(
        C.byref(shape), _p(cumulative_sequence_length), _p(past_seqlens), _p(block_table),
        _p(slot_mapping), int(rotary_positions), _p(flags), _s(stream))
    return _check(st, "pa_check_paged_indices", check)


def pa_kv_append_bnsh(shape, query, key, value, present_key, present_value,
                      total_sequence_length, key_total_sequence_lengths, cos_cache=None,
                      sin_cache=None, rotary_dim=0, rotary_mode=PA_ROTARY_NONE,
                      rotary_positions=0, stream=None, check=True):
    st = lib().pa_kv_append_bnsh(
        C.byref(shape), _p(query), _p(key), _p(value), _p(present_key), _p(present_value),
        _p(total_sequence_length), _p(key_total_sequence_lengths), _p(cos_cache), _p(sin_cache),
        int(rotary_dim), int(rotary_mode), int(rotary_positions), _s(stream))
    return _check(st, "pa_kv_append_bnsh", check)


def bnsh_shape(batch, seq_len, num_heads, kv_num_heads, head_size, max_cache_seq,
               packed_qkv=False):
    return BnshShape(batch, seq_len, num_heads, kv_num_heads, head_size, max_cache_seq,
                     int(bool(packed_qkv)))


def pa_timing_enable(on=True):
    lib().pa_timing_enable(int(bool(on)))


def pa_timing_reset():
    lib().pa_timing_reset()


def pa_timing_get(kernel=None):
    """(total milliseconds, launches) of the recorded launches of ``kernel`` (all if None)."""
    ms = C.c_double()
    n = C.c_int64()
    st = lib().pa_timing_get(kernel.encode() if kernel else None, C.byref(ms), C.byref(n))
    _check(st, "pa_timing_get", True)
    return ms.value, n.value
