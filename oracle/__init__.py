"""ctypes front end of the CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers. The HIP library does not import this module and this
module does not import the HIP library; they share only the seeded input generators.

Every function takes and returns numpy arrays in the layouts the C file documents. Inputs are
copied to C-contiguous arrays of the right dtype; fp16 data travels as its raw uint16 bits.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = C.POINTER(C.c_uint16)
_i32p = C.POINTER(C.c_int32)
_f32p = C.POINTER(C.c_float)
_vp = C.c_void_p
_i = C.c_int
_ll = C.c_longlong
_d = C.c_double


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # noqa: WPS433 (build on first use)
        _build.build()
    lib = C.CDLL(_LIB_PATH)
    lib.oracle_f16_to_f64.argtypes = [C.c_uint16]
    lib.oracle_f16_to_f64.restype = _d
    lib.oracle_f64_to_f16.argtypes = [_d]
    lib.oracle_f64_to_f16.restype = C.c_uint16
    lib.oracle_f32_to_f16.argtypes = [C.c_float]
    lib.oracle_f32_to_f16.restype = C.c_uint16
    lib.oracle_past_length_padded.argtypes = [_i, _i, _i]
    lib.oracle_past_length_padded.restype = _i
    lib.oracle_kv_append.argtypes = [_i] * 8 + [_vp] * 5 + [_vp] * 4 + [_vp, _vp, _i, _i]
    lib.oracle_kv_append.restype = None
    lib.oracle_rotate_query.argtypes = [_i] * 5 + [_vp] * 5 + [_i, _i, _vp]
    lib.oracle_rotate_query.restype = None
    lib.oracle_build_edges.argtypes = [_i] * 4 + [_vp] * 5
    lib.oracle_build_edges.restype = None
    lib.oracle_kv_append_bnsh.argtypes = [_i] * 7 + [_vp] * 5 + [_i, _vp, _vp, _vp, _i, _i, _i]
    lib.oracle_kv_append_bnsh.restype = None
    lib.oracle_paged_attention.argtypes = ([_i] * 7 + [_vp, _ll, _vp, _vp, _vp, _vp, _vp, _d, _i,
                                                       _vp])
    lib.oracle_paged_attention.restype = None
    lib.oracle_paged_attention_partials.argtypes = ([_i] * 7 + [_vp, _ll, _vp, _vp, _vp, _vp, _vp,
                                                                _d, _i, _i, _i, _vp, _vp, _vp])
    lib.oracle_paged_attention_partials.restype = None
    lib.oracle_split_combine.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
    lib.oracle_split_combine.restype = None
    lib.oracle_sparse_forward.argtypes = ([_i] * 7 + [_vp] * 5 + [_d, _vp, _vp, _vp, _vp])
    lib.oracle_sparse_forward.restype = None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(_vp)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _h(a):
    """fp16 array -> contiguous uint16 view of its bits."""
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


# -------------------------------------------------------------------------------------------
def f16_to_f64(bits):
    lib = _load()
    return np.array([lib.oracle_f16_to_f64(int(b)) for b in np.asarray(bits).reshape(-1)],
                    dtype=np.float64)


def f64_to_f16_bits(x):
    lib = _load()
    return np.array([lib.oracle_f64_to_f16(float(v)) for v in np.asarray(x).reshape(-1)],
                    dtype=np.uint16)


def f32_to_f16_bits(x):
    lib = _load()
    return np.array([lib.oracle_f32_to_f16(float(v))
                     for v in np.asarray(x, dtype=np.float32).reshape(-1)], dtype=np.uint16)


def past_length_padded(total_sequence_length, key_total_sequence_length, seq_len):
    return _load().oracle_past_length_padded(int(total_sequence_length),
                                             int(key_total_sequence_length), int(seq_len))


def kv_append(w, key_cache=None, value_cache=None):
    """Fused rotary + scatter of workload ``w``'s new rows. Returns updated (key_cache, value_cache)
    copies (fp16 [NB, bs, G, D]); the inputs are not modified."""
    lib = _load()
    kc = _h(w["key_cache"] if key_cache is None else key_cache).copy()
    vc = _h(w["value_cache"] if value_cache is None else value_cache).copy()
    q, k, v = _h(w["query"]), _h(w["key"]), _h(w["value"])
    cu, past, bt = _c(w["cu"], np.int32), _c(w["past"], np.int32), _c(w["block_table"], np.int32)
    sm = _c(w["slot_mapping"], np.int32)
    cs, sn = _h(w["cos"]), _h(w["sin"])
    lib.oracle_kv_append(w["T"], w["B"], w["H"], w["G"], w["D"], w["bs"], w["MB"],
                         int(w["packed"]), _p(q), _p(k), _p(v), _p(kc), _p(vc), _p(cu), _p(past),
                         _p(bt), _p(sm), _p(cs), _p(sn), int(w["rotary_dim"]),
                         int(w["rotary_mode"]))
    return kc.view(np.float16), vc.view(np.float16)


def rotate_query(w, rotary_mode=None, rotary_dim=None):
    """New query rows of workload ``w`` rotated at their positions (the key rotation applied to
    every query head). Returns fp16 [T, H*D]."""
    lib = _load()
    q = _h(w["query"])
    cu, past = _c(w["cu"], np.int32), _c(w["past"], np.int32)
    cs, sn = _h(w["cos"]), _h(w["sin"])
    out = np.zeros((w["T"], w["H"] * w["D"]), dtype=np.uint16)
    lib.oracle_rotate_query(w["B"], w["H"], w["G"], w["D"], int(w["packed"]), _p(q), _p(cu),
                            _p(past), _p(cs), _p(sn),
                            int(w["rotary_dim"] if rotary_dim is None else rotary_dim),
                            int(w["rotary_mode"] if rotary_mode is None else rotary_mode),
                            _p(out))
    return out.view(np.float16)


def kv_append_bnsh(bw):
    """The append page's pass over a contiguous BNSH cache for workload ``bw`` (see
    workloads.bnsh_workload). Returns updated (present_key, present_value) copies,
    fp16 [B, KVH, max_cache_seq, D]."""
    lib = _load()
    pk = _h(bw["present_key"]).copy()
    pv = _h(bw["present_value"]).copy()
    lib.oracle_kv_append_bnsh(bw["B"], bw["S"], bw["H"], bw["KVH"], bw["D"], bw["max_seq"],
                              int(bw["packed"]), _p(_h(bw["query"])), _p(_h(bw["key"])),
                              _p(_h(bw["value"])), _p(pk), _p(pv), int(bw["total_seq"]),
                              _p(_c(bw["key_total"], np.int32)), _p(_h(bw["cos"])),
                              _p(_h(bw["sin"])), int(bw["rotary_dim"]), int(bw["rotary_mode"]),
                              int(bw["rotary_positions"]))
    return pk.view(np.float16), pv.view(np.float16)


def build_edges(mask, q_batch, used_kv_lens, block_size):
    """Edge list from a kept-block mask [tq, hkv, nblk]: (edge_meta [E, 5] int32,
    group_ptr [tq*hkv + 1] int32)."""
    lib = _load()
    mk = np.ascontiguousarray(mask != 0, dtype=np.uint8)
    tq, hkv, nblk = mk.shape
    E = int(mk.sum())
    em = np.zeros((max(E, 1), 5), dtype=np.int32)
    gp = np.zeros(tq * hkv + 1, dtype=np.int32)
    lib.oracle_build_edges(tq, hkv, nblk, int(block_size), _p(mk), _p(_c(q_batch, np.int32)),
                           _p(_c(used_kv_lens, np.int32)), _p(em), _p(gp))
    return em[:E], gp


def _q_stride(w):
    return (w["H"] + 2 * w["G"]) * w["D"] if w["packed"] else w["H"] * w["D"]


def paged_attention(w, key_cache=None, value_cache=None, causal=None, scale=None):
    """Dense paged attention of workload ``w`` over the given caches. Returns fp16 [T, H*D]."""
    lib = _load()
    kc = _h(w["key_cache"] if key_cache is None else key_cache)
    vc = _h(w["value_cache"] if value_cache is None else value_cache)
    q = _h(w["query"])
    cu, past, bt = _c(w["cu"], np.int32), _c(w["past"], np.int32), _c(w["block_table"], np.int32)
    out = np.zeros((w["T"], w["H"] * w["D"]), dtype=np.uint16)
    lib.oracle_paged_attention(w["T"], w["B"], w["H"], w["G"], w["D"], w["bs"], w["MB"], _p(q),
                               _q_stride(w), _p(kc), _p(vc), _p(cu), _p(past), _p(bt),
                               float(w["scale"] if scale is None else scale),
                               int(w["causal"] if causal is None else causal), _p(out))
    return out.view(np.float16)


def paged_attention_partials(w, num_splits, chunk_keys=0, key_cache=None, value_cache=None,
                             causal=None):
    """Split-KV partials. Returns (o [T*S*H, D], m [T*S*H], l [T*S*H]) float32 with
    p = (i*S + s)*H + h."""
    lib = _load()
    kc = _h(w["key_cache"] if key_cache is None else key_cache)
    vc = _h(w["value_cache"] if value_cache is None else value_cache)
    q = _h(w["query"])
    cu, past, bt = _c(w["cu"], np.int32), _c(w["past"], np.int32), _c(w["block_table"], np.int32)
    P = w["T"] * num_splits * w["H"]
    o = np.zeros((P, w["D"]), dtype=np.float32)
    m = np.zeros(P, dtype=np.float32)
    l = np.zeros(P, dtype=np.float32)
    lib.oracle_paged_attention_partials(
        w["T"], w["B"], w["H"], w["G"], w["D"], w["bs"], w["MB"], _p(q), _q_stride(w), _p(kc),
        _p(vc), _p(cu), _p(past), _p(bt), float(w["scale"]),
        int(w["causal"] if causal is None else causal), int(num_splits), int(chunk_keys),
        _p(o), _p(m), _p(l))
    return o, m, l


def split_combine(o, m, l, *, lanes, head_dim, group_ptr=None, num_groups=None, num_splits=0,
                  out_dtype=np.float16):
    """LSE merge. Returns [num_groups*lanes, head_dim] of out_dtype (fp16 or float32)."""
    lib = _load()
    o, m, l = _c(o, np.float32), _c(m, np.float32), _c(l, np.float32)
    gp = _c(group_ptr, np.int32)
    if num_groups is None:
        num_groups = (len(gp) - 1) if gp is not None else (m.size // (lanes * num_splits))
    is16 = np.dtype(out_dtype) == np.float16
    out = np.zeros((num_groups * lanes, head_dim), dtype=np.uint16 if is16 else np.float32)
    lib.oracle_split_combine(_p(o), _p(m), _p(l), _p(gp), int(num_groups), int(lanes),
                             int(num_splits), int(head_dim), 0 if is16 else 1, _p(out))
    return out.view(np.float16) if is16 else out


def sparse_forward(sw, edge_meta=None, block_tables=None, q_pos=None):
    """Block-sparse edge forward of sparse workload ``sw``. Returns (o [E*qhead, D], m, l).
    ``q_pos`` (int32 [Tq]) adds the causal mask: key position > q_pos[q_idx] is excluded."""
    lib = _load()
    em = _c(sw["edge_meta"] if edge_meta is None else edge_meta, np.int32)
    bt = _c(sw["block_tables"] if block_tables is None else block_tables, np.int32)
    E = em.shape[0]
    P = E * sw["qhead"]
    o = np.zeros((P, sw["D"]), dtype=np.float32)
    m = np.zeros(P, dtype=np.float32)
    l = np.zeros(P, dtype=np.float32)
    lib.oracle_sparse_forward(E, sw["hkv"], sw["qhead"], sw["D"], sw["block_size"],
                              sw["page_size"], sw["max_pages"], _p(_c(sw["q_buf"], np.float32)),
                              _p(_c(sw["k_pages"], np.float32)),
                              _p(_c(sw["v_pages"], np.float32)), _p(em), _p(bt),
                              float(sw["softmax_scale"]), _p(_c(q_pos, np.int32)), _p(o),
                              _p(m), _p(l))
    return o, m, l
