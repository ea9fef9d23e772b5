"""Device-side marshalling for the seeded workloads: copy a workload's arrays to the GPU and call
the C entry points with the right shapes and workspaces. No arithmetic of the method lives here;
torch provides device memory and the stream only.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (PA_F16, PA_F32, PA_SPLITS_AUTO, bnsh_shape, pa_append_attention,
               pa_check_paged_indices, pa_kv_append, pa_kv_append_bnsh, pa_kv_append_rotate_query,
               pa_paged_attention,
               pa_paged_attention_workspace_size, pa_sparse_build_edges,
               pa_sparse_build_edges_workspace_size, pa_sparse_forward, pa_sparse_forward_causal,
               pa_sparse_forward_workspace_size, pa_split_combine, paged_shape, sparse_shape)


def to_dev(a, device="cuda"):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def workspace(nbytes, device="cuda"):
    """A 256-byte aligned device buffer of at least nbytes (torch allocations are aligned)."""
    return torch.empty(max(256, int(nbytes)), dtype=torch.uint8, device=device)


class PagedCase:
    """A paged workload resident on the device."""

    def __init__(self, w, device="cuda"):
        self.w = w
        self.device = device
        self.shape = paged_shape(w["B"], w["T"], w["H"], w["G"], w["D"], w["NB"], w["bs"],
                                 w["MB"], w["packed"])
        self.query = to_dev(w["query"], device)
        self.key = to_dev(w["key"], device)
        self.value = to_dev(w["value"], device)
        self.key_cache = to_dev(w["key_cache"], device)
        self.value_cache = to_dev(w["value_cache"], device)
        self.cu = to_dev(w["cu"], device)
        self.past = to_dev(w["past"], device)
        self.block_table = to_dev(w["block_table"], device)
        self.slot_mapping = to_dev(w["slot_mapping"], device)
        self.cos = to_dev(w["cos"], device)
        self.sin = to_dev(w["sin"], device)
        self.output = torch.empty((w["T"], w["H"] * w["D"]), dtype=torch.float16, device=device)
        self._ws = {}

    def check_indices(self, use_slot_mapping=True, use_block_table=True, stream=None):
        """The device check of this workload's index arrays (pa_check_paged_indices); waits for
        it and returns the PA_CHECK_* flag word (0: every rule holds)."""
        flags = torch.full((1,), -1, dtype=torch.int32, device=self.device)
        rot = 0 if self.cos is None else self.cos.shape[0]
        pa_check_paged_indices(self.shape, self.cu, self.past,
                               self.block_table if use_block_table else None,
                               self.slot_mapping if use_slot_mapping else None, flags,
                               rotary_positions=rot, stream=stream)
        torch.cuda.synchronize()
        return int(flags.item())

    def append(self, use_slot_mapping=True, stream=None):
        w = self.w
        pa_kv_append(self.shape, self.query if w["packed"] else None, self.key, self.value,
                     self.key_cache, self.value_cache, self.cu, self.past, self.block_table,
                     self.slot_mapping if use_slot_mapping else None, self.cos, self.sin,
                     w["rotary_dim"], w["rotary_mode"],
                     0 if self.cos is None else self.cos.shape[0], stream=stream)

    def append_rotate_query(self, q_out=None, use_slot_mapping=True, stream=None):
        """The append plus every new query row rotated at its position into q_out
        (fp16 [T, H*D]; allocated when not given). Returns q_out."""
        w = self.w
        if q_out is None:
            q_out = torch.empty((w["T"], w["H"] * w["D"]), dtype=torch.float16,
                                device=self.device)
        pa_kv_append_rotate_query(
            self.shape, self.query, None if w["packed"] else self.key,
            None if w["packed"] else self.value, self.key_cache, self.value_cache, self.cu,
            self.past, self.block_table, q_out,
            self.slot_mapping if use_slot_mapping else None, self.cos, self.sin,
            w["rotary_dim"], w["rotary_mode"], 0 if self.cos is None else self.cos.shape[0],
            stream=stream)
        return q_out

    def workspace_for(self, num_splits):
        n = pa_paged_attention_workspace_size(self.shape, num_splits)
        if num_splits not in self._ws or self._ws[num_splits].numel() < n:
            self._ws[num_splits] = workspace(n, self.device)
        return self._ws[num_splits], n

    def attention(self, num_splits=PA_SPLITS_AUTO, causal=None, scale=None, out=None,
                  stream=None):
        w = self.w
        ws, n = self.workspace_for(num_splits)
        out = self.output if out is None else out
        pa_paged_attention(self.shape, self.query, self.key_cache, self.value_cache, self.cu,
                           self.past, self.block_table,
                           w["scale"] if scale is None else scale,
                           w["causal"] if causal is None else causal, num_splits, ws, n, out,
                           stream=stream)
        return out

    def append_attention(self, num_splits=PA_SPLITS_AUTO, q_out=None, use_slot_mapping=True,
                         causal=None, scale=None, out=None, stream=None):
        """The append and the attention in one call (pa_append_attention). With q_out
        (fp16 [T, H*D]) the query rows are rotated into it and the attention reads them."""
        w = self.w
        ws, n = self.workspace_for(num_splits)
        out = self.output if out is None else out
        pa_append_attention(
            self.shape, self.query, self.key, self.value, self.key_cache, self.value_cache,
            self.cu, self.past, self.block_table, w["scale"] if scale is None else scale,
            w["causal"] if causal is None else causal, num_splits, ws, n, out,
            slot_mapping=self.slot_mapping if use_slot_mapping else None, cos_cache=self.cos,
            sin_cache=self.sin, rotary_dim=w["rotary_dim"], rotary_mode=w["rotary_mode"],
            rotary_positions=0 if self.cos is None else self.cos.shape[0], q_out=q_out,
            stream=stream)
        return out


class SparseCase:
    """A block-sparse workload resident on the device."""

    def __init__(self, sw, device="cuda"):
        self.sw = sw
        self.device = device
        self.shape = sparse_shape(sw["E"], sw["Tq"], sw["hkv"], sw["qhead"], sw["D"],
                                  sw["block_size"], sw["page_size"], sw["num_pages"],
                                  sw["max_pages"], sw["batch"])
        self.q = to_dev(sw["q_buf"], device)
        self.k = to_dev(sw["k_pages"], device)
        self.v = to_dev(sw["v_pages"], device)
        self.edge_meta = to_dev(sw["edge_meta"], device)
        self.block_tables = to_dev(sw["block_tables"], device)
        self.group_ptr = to_dev(sw["group_ptr"], device)
        P = sw["E"] * sw["qhead"]
        self.o = torch.empty((P, sw["D"]), dtype=torch.float32, device=device)
        self.m = torch.empty(P, dtype=torch.float32, device=device)
        self.l = torch.empty(P, dtype=torch.float32, device=device)
        self.out = torch.empty((sw["Tq"] * sw["hkv"] * sw["qhead"], sw["D"]),
                               dtype=torch.float32, device=device)
        n = pa_sparse_forward_workspace_size(self.shape)
        self.ws = workspace(n, device)
        self.ws_bytes = n
        self.q_pos = None

    def forward(self, causal=False, stream=None):
        """Partials of every edge; causal=True masks keys past each row's q_pos."""
        sw = self.sw
        if causal:
            if self.q_pos is None:
                self.q_pos = to_dev(sw["q_pos"], self.device)
            pa_sparse_forward_causal(self.shape, self.q, self.k, self.v, self.edge_meta,
                                     self.block_tables, self.q_pos, sw["softmax_scale"],
                                     self.ws, self.ws_bytes, self.o, self.m, self.l,
                                     stream=stream)
        else:
            pa_sparse_forward(self.shape, self.q, self.k, self.v, self.edge_meta,
                              self.block_tables, sw["softmax_scale"], 0, self.ws, self.ws_bytes,
                              self.o, self.m, self.l, stream=stream)
        return self.o, self.m, self.l

    def combine(self, out_dtype=PA_F32, out=None, stream=None):
        sw = self.sw
        out = self.out if out is None else out
        pa_split_combine(self.o, self.m, self.l, self.group_ptr, sw["Tq"] * sw["hkv"],
                         sw["qhead"], 0, sw["D"], out_dtype, out, stream=stream)
        return out


class BnshCase:
    """A contiguous-cache (BNSH) append workload resident on the device."""

    def __init__(self, bw, device="cuda"):
        self.bw = bw
        self.device = device
        self.shape = bnsh_shape(bw["B"], bw["S"], bw["H"], bw["KVH"], bw["D"], bw["max_seq"],
                                bw["packed"])
        self.query = to_dev(bw["query"], device)
        self.key = to_dev(bw["key"], device)
        self.value = to_dev(bw["value"], device)
        self.present_key = to_dev(bw["present_key"], device)
        self.present_value = to_dev(bw["present_value"], device)
        self.total = to_dev(np.array([bw["total_seq"]], dtype=np.int32), device)
        self.key_total = to_dev(bw["key_total"].astype(np.int32), device)
        self.cos = to_dev(bw["cos"], device)
        self.sin = to_dev(bw["sin"], device)

    def append(self, stream=None):
        bw = self.bw
        pa_kv_append_bnsh(self.shape, self.query, self.key, self.value, self.present_key,
                          self.present_value, self.total, self.key_total, self.cos, self.sin,
                          bw["rotary_dim"], bw["rotary_mode"], bw["rotary_positions"],
                          stream=stream)
        return self.present_key, self.present_value


class EdgeBuilder:
    """A sparse workload's kept-block mask on the device, turned into (edge_meta, group_ptr)."""

    def __init__(self, sw, capacity=None, device="cuda"):
        self.sw = sw
        self.mask = to_dev(np.ascontiguousarray(sw["block_mask"], dtype=np.uint8), device)
        self.q_batch = to_dev(sw["q_batch"].astype(np.int32), device)
        self.used = to_dev(sw["used_kv_lens"].astype(np.int32), device)
        tq, hkv, nblk = sw["block_mask"].shape
        self.dims = (tq, hkv, nblk)
        self.capacity = tq * hkv * nblk if capacity is None else capacity
        self.edge_meta = torch.empty((max(1, self.capacity), 5), dtype=torch.int32,
                                     device=device)
        self.group_ptr = torch.empty(tq * hkv + 1, dtype=torch.int32, device=device)
        n = pa_sparse_build_edges_workspace_size(tq, hkv)
        self.ws = workspace(n, device)
        self.ws_bytes = n

    def build(self, stream=None):
        tq, hkv, nblk = self.dims
        pa_sparse_build_edges(tq, hkv, nblk, self.sw["block_size"], self.sw["batch"], self.mask,
                              self.q_batch, self.used, self.capacity, self.edge_meta,
                              self.group_ptr, self.ws, self.ws_bytes, stream=stream)
        return self.edge_meta, self.group_ptr


def combine(o, m, l, *, lanes, head_dim, group_ptr=None, num_groups=None, num_splits=0,
            out_dtype=PA_F16, device="cuda"):
    """pa_split_combine on host arrays copied to the device; returns a device tensor."""
    od, md, ld = to_dev(o, device), to_dev(m, device), to_dev(l, device)
    gp = to_dev(group_ptr, device) if group_ptr is not None else None
    if num_groups is None:
        num_groups = (len(group_ptr) - 1) if group_ptr is not None else m.size // (lanes * num_splits)
    dt = torch.float16 if out_dtype == PA_F16 else torch.float32
    out = torch.empty((num_groups * lanes, head_dim), dtype=dt, device=device)
    pa_split_combine(od, md, ld, gp, num_groups, lanes, num_splits, head_dim, out_dtype, out)
    return out
