"""Seeded synthetic inputs for the paged-attention path.

These generators only draw inputs: tensor contents, sequence lengths, block tables, slot
mappings, rotary tables and block-sparse edge lists, with the shapes and value distributions of
the five workloads the pages' kernels are sized for. They hold none of the attention, rotary or
merge arithmetic. The CPU oracle and the HIP library both consume what they return.

Every generator takes a seed and draws from ``numpy.random.default_rng(seed)`` in the order its
docstring lists, so a workload is reproducible from its name and seed alone.

Layouts (the pages' PagedAttention manifest, "inputs"/"outputs" blocks):
  query        fp16 [T, H*D]            or packed [T, (H+2G)*D] as Q | K | V per row
  key, value   fp16 [T, G*D]            (None when packed)
  key_cache    fp16 [NB, bs, G, D]      value_cache the same shape
  cu           int32 [B+1]              cumulative_sequence_length
  past         int32 [B]                past_seqlens
  block_table  int32 [B, MB]            -1 marks an entry no sequence uses
  slot_mapping int32 [T] or None
  cos, sin     fp16 [P, R/2] or None
"""
from __future__ import annotations

import math

import numpy as np

ROTARY_NONE = 0
ROTARY_NEOX = 1
ROTARY_INTERLEAVED = 2

_CHUNK = 1 << 22  # elements drawn per call when filling large tensors


def _fill_normal(rng, shape, dtype, scale=1.0):
    """float32 standard normals (times ``scale``), cast to ``dtype``, drawn in row-major chunks."""
    out = np.empty(shape, dtype=dtype)
    flat = out.reshape(-1)
    buf = np.empty(min(_CHUNK, max(1, flat.size)), dtype=np.float32)
    for start in range(0, flat.size, _CHUNK):
        n = min(_CHUNK, flat.size - start)
        rng.standard_normal(out=buf[:n], dtype=np.float32)
        if scale != 1.0:
            buf[:n] *= np.float32(scale)
        flat[start:start + n] = buf[:n]
    return out


def rotary_tables(positions: int, rotary_dim: int, theta: float = 10000.0):
    """cos/sin tables [positions, rotary_dim/2]: angle pos * theta^(-2i/R), float64, then fp16 (RNE).

    The pages index the tables as position * (R/2) + slot and give no rule for their values;
    this is the usual rotary frequency ladder.
    """
    half = rotary_dim // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
    ang = np.arange(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float16), np.sin(ang).astype(np.float16)


def paged_workload(seed, *, past, n_new, num_heads, kv_num_heads, head_size, block_size,
                   table="pool", slack=0.10, max_blocks=None, packed=False,
                   rotary_mode=ROTARY_NONE, rotary_dim=0, rotary_positions=None,
                   theta=10000.0, key_scale=1.0, use_slot_mapping=False, causal=1,
                   scale=None, poison=False, key_step=None, name="paged"):
    """Generic paged workload.

    ``past`` and ``n_new`` are either integer sequences (used as given) or callables
    ``f(rng) -> array`` drawn first, in that order. Draw order after the lengths:
      1. the physical block assignment (a permutation),
      2. key_cache, 3. value_cache (whole pool, every block),
      4. new rows: packed QKV [T, (H+2G)D], or query [T, H*D] then key then value [T, G*D].
    Keys (cache and new) are multiplied by ``key_scale`` before the fp16 cast.

    table == "dense": NB = B * MB and block_table = permutation(NB).reshape(B, MB).
    table == "pool":  NB = ceil((1 + slack) * sum_b ceil(L_b / bs)); each sequence takes the next
                      ceil(L_b / bs) ids of permutation(NB), in batch order; unused entries are -1.
    poison=True writes fp16 NaN into every cache row a sequence does not own below L_b
    (rows at positions >= L_b of owned blocks, and every block no sequence owns).
    key_step: a list of (position, factor) pairs; every key of a sequence at absolute position
    >= position (cache rows below past, new rows above it) is multiplied by factor (float32,
    then fp16), the pairs compounding. It draws nothing: scores that jump by a known amount
    partway through a sequence.
    """
    rng = np.random.default_rng(seed)
    past = np.asarray(past(rng) if callable(past) else past, dtype=np.int64)
    n_new = np.asarray(n_new(rng) if callable(n_new) else n_new, dtype=np.int64)
    if n_new.ndim == 0:
        n_new = np.full(past.shape, int(n_new), dtype=np.int64)
    B = past.shape[0]
    H, G, D, bs = num_heads, kv_num_heads, head_size, block_size
    L = past + n_new
    need = (L + bs - 1) // bs
    MB = int(max_blocks) if max_blocks is not None else int(max(1, need.max()))
    if need.max() > MB:
        raise ValueError("max_blocks too small for the longest sequence")

    if table == "dense":
        NB = B * MB
        block_table = rng.permutation(NB).astype(np.int32).reshape(B, MB)
    elif table == "pool":
        total = int(need.sum())
        NB = int(math.ceil((1.0 + slack) * total))
        perm = rng.permutation(NB).astype(np.int32)
        block_table = np.full((B, MB), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            block_table[b, :need[b]] = perm[off:off + need[b]]
            off += int(need[b])
    else:
        raise ValueError(table)

    key_cache = _fill_normal(rng, (NB, bs, G, D), np.float16, key_scale)
    value_cache = _fill_normal(rng, (NB, bs, G, D), np.float16)

    T = int(n_new.sum())
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(n_new)
    if packed:
        query = _fill_normal(rng, (T, (H + 2 * G) * D), np.float16)
        if key_scale != 1.0:
            ks = query[:, H * D:(H + G) * D].astype(np.float32) * np.float32(key_scale)
            query[:, H * D:(H + G) * D] = ks.astype(np.float16)
        key = value = None
    else:
        query = _fill_normal(rng, (T, H * D), np.float16)
        key = _fill_normal(rng, (T, G * D), np.float16, key_scale)
        value = _fill_normal(rng, (T, G * D), np.float16)

    if key_step:
        for b in range(B):
            f = np.ones(int(L[b]), dtype=np.float32)
            for pos0, fac in key_step:
                f[int(pos0):] *= np.float32(fac)
            for j in range(int(L[b])):
                if f[j] == 1.0:
                    continue
                if j < past[b]:
                    blk, off = int(block_table[b, j // bs]), j % bs
                    key_cache[blk, off] = (key_cache[blk, off].astype(np.float32)
                                           * f[j]).astype(np.float16)
                else:
                    i = int(cu[b]) + j - int(past[b])
                    if packed:
                        ks = query[i, H * D:(H + G) * D]
                        query[i, H * D:(H + G) * D] = (ks.astype(np.float32) * f[j]).astype(
                            np.float16)
                    else:
                        key[i] = (key[i].astype(np.float32) * f[j]).astype(np.float16)

    slot_mapping = None
    if use_slot_mapping:
        # The slot recipe the rotary-append workload states: bt[b][pos/bs]*bs + pos%bs.
        slot_mapping = np.empty(T, dtype=np.int32)
        for b in range(B):
            for t in range(int(n_new[b])):
                pos = int(past[b]) + t
                slot_mapping[cu[b] + t] = block_table[b, pos // bs] * bs + pos % bs

    cos = sin = None
    if rotary_mode != ROTARY_NONE:
        P = int(rotary_positions) if rotary_positions is not None else int(L.max())
        cos, sin = rotary_tables(P, rotary_dim, theta)

    if poison:
        nan = np.float16(np.nan)
        owned = np.zeros(NB, dtype=bool)
        for b in range(B):
            for j in range(int(need[b])):
                blk = int(block_table[b, j])
                owned[blk] = True
                lo = max(0, int(L[b]) - j * bs)
                if lo < bs:
                    key_cache[blk, lo:] = nan
                    value_cache[blk, lo:] = nan
        key_cache[~owned] = nan
        value_cache[~owned] = nan

    return dict(
        name=name, seed=seed, B=B, T=T, H=H, G=G, D=D, bs=bs, NB=NB, MB=MB,
        query=query, key=key, value=value, packed=bool(packed),
        key_cache=key_cache, value_cache=value_cache,
        cu=cu, past=past.astype(np.int32), block_table=block_table, slot_mapping=slot_mapping,
        cos=cos, sin=sin, rotary_dim=int(rotary_dim) if rotary_mode else 0,
        rotary_mode=int(rotary_mode),
        scale=float(scale) if scale is not None else 1.0 / math.sqrt(D),
        causal=int(causal),
    )


def tiny_decode(seed=0):
    """Tiny paged decode: B=2, H=4, G=2, D=64, bs=16, 16 blocks by seeded permutation,
    past={37,100}, one new token each, causal, fp16 N(0,1), scale 1/8, no rotary."""
    return paged_workload(seed, past=[37, 100], n_new=1, num_heads=4, kv_num_heads=2,
                          head_size=64, block_size=16, table="dense", max_blocks=8,
                          scale=1.0 / 8.0, name="tiny_decode_b2_h4g2_d64")


def rotary_append_decode(seed=1, rotary_mode=ROTARY_NEOX):
    """Rotary KV append + decode: B=4, H=G=8, D=128, R=128, bs=32, 512 blocks by permutation,
    past ~ U[0, 4095), one new token each, cos/sin for positions < 4096 (theta 1e4),
    slot_mapping = bt[b][pos/32]*32 + pos%32, separate key/value."""
    tag = "neox" if rotary_mode == ROTARY_NEOX else "interleaved"
    return paged_workload(seed, past=lambda r: r.integers(0, 4095, size=4), n_new=1,
                          num_heads=8, kv_num_heads=8, head_size=128, block_size=32,
                          table="dense", max_blocks=128, rotary_mode=rotary_mode,
                          rotary_dim=128, rotary_positions=4096, use_slot_mapping=True,
                          name=f"rotary_append_decode_{tag}_b4_h8_d128")


def gqa_decode(seed=2, batch=64):
    """GQA serving decode: B=64, H=32, G=8, D=128, bs=16, past ~ U[512, 8192] (inclusive),
    one new token each, pool of sum ceil(L/16) blocks + 10% slack, shuffled, keys x0.5."""
    return paged_workload(seed, past=lambda r: r.integers(512, 8193, size=batch), n_new=1,
                          num_heads=32, kv_num_heads=8, head_size=128, block_size=16,
                          table="pool", slack=0.10, max_blocks=513, key_scale=0.5,
                          name=f"gqa_decode_b{batch}_h32g8_d128_bs16")


def mixed_prefill_decode(seed=3, prefill_tokens=512, n_prefill=8, n_decode=56):
    """Mixed chunked prefill + decode: 8 sequences of 512 new tokens on past ~ U[0, 2048], then 56
    sequences of 1 token on past ~ U[256, 16384]; H=32, G=8, D=128, bs=32, packed QKV,
    NeoX rotary on all 128 dims, pool + 10% slack."""
    def past(r):
        return np.concatenate([r.integers(0, 2049, size=n_prefill),
                               r.integers(256, 16385, size=n_decode)])
    n_new = np.array([prefill_tokens] * n_prefill + [1] * n_decode)
    return paged_workload(seed, past=past, n_new=n_new, num_heads=32, kv_num_heads=8,
                          head_size=128, block_size=32, table="pool", slack=0.10,
                          max_blocks=513, packed=True, rotary_mode=ROTARY_NEOX, rotary_dim=128,
                          rotary_positions=16385,
                          name=f"mixed_prefill{n_prefill}x{prefill_tokens}_decode{n_decode}")


def append_stress(seed=5):
    """KV-append bandwidth run: the mixed workload's shapes (H=32, G=8, D=128, bs=32, packed
    QKV, NeoX rotary on all 128 dims) with 16x its prefill tokens (8 sequences x 8192 new tokens
    on past ~ U[0, 2048]) and no decode rows: T = 65536, about 554 MB moved by the append."""
    return mixed_prefill_decode(seed, prefill_tokens=8192, n_prefill=8, n_decode=0)


def bnsh_workload(seed, *, batch, seq_len, num_heads, kv_num_heads, head_size, max_seq,
                  key_total, total_seq=None, packed=False, rotary_mode=ROTARY_NONE,
                  rotary_dim=None, rotary_positions=None, theta=10000.0, name="bnsh"):
    """The append page's own layout: new rows in a padded batch [B, seq_len] and a contiguous
    BNSH cache [B, KVH, max_seq, D] (present_key / present_value, filled with N(0,1)).

    key_total: per-batch total sequence lengths (a list, or a callable of the generator);
    total_seq: the scalar total_sequence_length (defaults to max(key_total); equal to seq_len
    makes the call a prompt, where every row's past length is 0).
    Draw order: key_total (when callable); present_key; present_value; the new rows.
    """
    rng = np.random.default_rng(seed)
    B, S, H, KVH, D = batch, seq_len, num_heads, kv_num_heads, head_size
    kt = np.asarray(key_total(rng) if callable(key_total) else key_total, dtype=np.int32)
    total = int(kt.max()) if total_seq is None else int(total_seq)
    present_key = _fill_normal(rng, (B, KVH, max_seq, D), np.float16)
    present_value = _fill_normal(rng, (B, KVH, max_seq, D), np.float16)
    if packed:
        query = _fill_normal(rng, (B * S, (H + 2 * KVH) * D), np.float16)
        key = value = None
    else:
        query = None
        key = _fill_normal(rng, (B * S, KVH * D), np.float16)
        value = _fill_normal(rng, (B * S, KVH * D), np.float16)
    cos = sin = None
    R = 0
    P = 0
    if rotary_mode != ROTARY_NONE:
        R = D if rotary_dim is None else rotary_dim
        P = max_seq if rotary_positions is None else rotary_positions
        cos, sin = rotary_tables(P, R, theta)
    return dict(name=name, seed=seed, B=B, S=S, H=H, KVH=KVH, D=D, max_seq=max_seq,
                packed=packed, query=query, key=key, value=value, present_key=present_key,
                present_value=present_value, total_seq=total, key_total=kt, cos=cos, sin=sin,
                rotary_dim=R, rotary_mode=rotary_mode, rotary_positions=P)


def bnsh_append(seed=6):
    """Contiguous-cache append at the mixed workload's prefill shape: 8 sequences x 512 new
    tokens of one padded batch, H=32, KVH=8, D=128, packed QKV, NeoX rotary on all dims, cache
    [8, 8, 4096, 128] per K and V, per-batch totals ~ U[512, 2560] (past = total - 512)."""
    return bnsh_workload(seed, batch=8, seq_len=512, num_heads=32, kv_num_heads=8,
                         head_size=128, max_seq=4096,
                         key_total=lambda r: r.integers(512, 2561, size=8), packed=True,
                         rotary_mode=ROTARY_NEOX, rotary_dim=128, rotary_positions=4096,
                         name="bnsh_b8_s512_h32kv8_d128")


# --------------------------------------------------------------------------------------------
# Block-sparse "edge" workloads (the fp32 KV-outer forward page).
# --------------------------------------------------------------------------------------------

def sparse_workload(seed, *, Tq, hkv, qhead, head_dim, block_size, page_size, batch,
                    key_capacity, window=4, p_random=0.05, unmapped_frac=0.10,
                    all_blocks=False, softmax_scale=None, outliers=None, tiny=None,
                    name="sparse"):
    """Block-sparse edge workload, fp32.

    Draw order: used_kv_lens = key_capacity - U{1..63} (clamped to >= 1) per batch; the page
    permutation; the unmapped table positions (exactly round(frac * entries), without
    replacement); k_pages; v_pages; q_buf; the Bernoulli block draws.

    Queries: Tq in total, Tq/batch per batch, right-aligned so that query j of batch b sits at key
    position used_b - Tq/batch + j. For each (q, h) the kept blocks are: the block holding that
    position and the window-1 blocks before it, block 0, and each other block below
    ceil(used_b / block_size) with probability p_random (all blocks if all_blocks).
    Edges (q_idx, h, blk, batch, block_len) are sorted by (q_idx, h, blk), with
    block_len = clamp(used_b - blk * block_size, 0, block_size) as the page's host does.
    group_ptr[q * hkv + h] is the CSR offset of that (q, h) group's first edge. q_pos[q] is that
    right-aligned key position (the causal limit when the mask is applied). block_mask
    [Tq, hkv, nblk] (uint8) and q_batch [Tq] are the kept-block mask and each row's batch, the
    inputs an edge-list builder turns into edge_meta and group_ptr.

    Wide-range options, drawn after everything above (the other draws do not change):
      outliers = (n, k_factor, v_factor): n channels (drawn without replacement) of every key
        row are multiplied by k_factor and of every value row by v_factor; the same query
        channels are divided by k_factor, so those channels' score terms keep unit scale while
        each key row spans the factor's range.
      tiny = (frac, factor): each (page, head, row) key/value row with probability frac, then
        each (query row, head) with probability frac, is multiplied by factor.
    """
    rng = np.random.default_rng(seed)
    ppb = block_size // page_size
    nblk = key_capacity // block_size
    max_pages = key_capacity // page_size
    num_pages = batch * max_pages
    hq = hkv * qhead
    qpb = Tq // batch
    used = np.maximum(1, key_capacity - rng.integers(1, 64, size=batch)).astype(np.int64)
    block_tables = rng.permutation(num_pages).astype(np.int32).reshape(batch, max_pages)
    n_unmapped = int(round(unmapped_frac * block_tables.size))
    if n_unmapped:
        idx = rng.choice(block_tables.size, size=n_unmapped, replace=False)
        block_tables.reshape(-1)[idx] = -1
    k_pages = _fill_normal(rng, (num_pages, hkv, page_size, head_dim), np.float32)
    v_pages = _fill_normal(rng, (num_pages, hkv, page_size, head_dim), np.float32)
    q_buf = _fill_normal(rng, (Tq, hq, head_dim), np.float32)

    nused = (used + block_size - 1) // block_size
    keep = np.zeros((Tq, hkv, nblk), dtype=bool)
    if all_blocks:
        for q in range(Tq):
            keep[q, :, :nused[q // qpb]] = True
    else:
        rnd = rng.random(size=(Tq, hkv, nblk)) < p_random
        for q in range(Tq):
            b = q // qpb
            pos = int(used[b]) - qpb + (q % qpb)
            qb = max(0, pos) // block_size
            k = keep[q]
            k[:, :nused[b]] = rnd[q, :, :nused[b]]
            k[:, max(0, qb - window + 1):qb + 1] = True
            k[:, 0] = True
    if outliers:
        n_ch, kf, vf = outliers
        ch = rng.choice(head_dim, size=int(n_ch), replace=False)
        k_pages[..., ch] *= np.float32(kf)
        v_pages[..., ch] *= np.float32(vf)
        q_buf[..., ch] /= np.float32(kf)
    if tiny:
        frac, fac = tiny
        rows = rng.random(size=k_pages.shape[:3]) < frac
        k_pages[rows] *= np.float32(fac)
        v_pages[rows] *= np.float32(fac)
        qrows = rng.random(size=q_buf.shape[:2]) < frac
        q_buf[qrows] *= np.float32(fac)
    q_pos = (used[np.arange(Tq) // qpb] - qpb + np.arange(Tq) % qpb).astype(np.int32)
    qi, hi, bi = np.nonzero(keep)          # row-major: already sorted by (q, h, blk)
    bb = qi // qpb
    blen = np.clip(used[bb] - bi * block_size, 0, block_size)
    edge_meta = np.stack([qi, hi, bi, bb, blen], axis=1).astype(np.int32)
    counts = keep.sum(axis=2).reshape(-1)
    group_ptr = np.zeros(Tq * hkv + 1, dtype=np.int32)
    group_ptr[1:] = np.cumsum(counts)
    return dict(
        name=name, seed=seed, Tq=Tq, hkv=hkv, qhead=qhead, hq=hq, D=head_dim,
        block_size=block_size, page_size=page_size, pages_per_block=ppb, batch=batch,
        num_pages=num_pages, max_pages=max_pages, used_kv_lens=used.astype(np.int32),
        q_buf=q_buf, k_pages=k_pages, v_pages=v_pages, block_tables=block_tables,
        edge_meta=edge_meta, group_ptr=group_ptr, E=int(edge_meta.shape[0]), q_pos=q_pos,
        block_mask=keep.astype(np.uint8), q_batch=(np.arange(Tq) // qpb).astype(np.int32),
        nblk=nblk,
        softmax_scale=float(softmax_scale) if softmax_scale is not None
        else 1.0 / math.sqrt(head_dim),
        causal=0,
    )


def block_sparse_forward(seed=4):
    """Block-sparse KV-outer fp32 forward: Tq=4096 (2048 per batch), hkv=8, qhead=4, D=128,
    block 64, page 16, key capacity 32768 per batch, batch=2; window of 4 blocks + block 0 +
    5% random; 10% of table entries unmapped; softmax_scale 1/sqrt(128), no causal mask."""
    return sparse_workload(seed, Tq=4096, hkv=8, qhead=4, head_dim=128, block_size=64,
                           page_size=16, batch=2, key_capacity=32768,
                           name="block_sparse_tq4096_hkv8_q4_d128_blk64")


def random_partials(seed, *, groups, lanes, head_dim, max_units=9, p_empty=0.1,
                    uniform_splits=0):
    """Seeded (o, m, l) partial sets for merge tests. With uniform_splits = S > 0 every group
    owns S units and group_ptr is None; otherwise group k owns U[0, max_units] units (some groups
    none) and group_ptr is their CSR offsets. Unit e holds `lanes` partials p = e*lanes + lane:
    o ~ N(0, 1) [P, head_dim] float32, m ~ U[-20, 20], l ~ U[0.5, 50]; a fraction p_empty of the
    partials are empty key ranges (o = 0, m = -1e30, l = 0)."""
    r = np.random.default_rng(seed)
    if uniform_splits > 0:
        counts = np.full(groups, uniform_splits, dtype=np.int64)
        gp = None
    else:
        counts = r.integers(0, max_units + 1, size=groups)
        gp = np.zeros(groups + 1, dtype=np.int32)
        gp[1:] = np.cumsum(counts)
    P = int(counts.sum()) * lanes
    o = r.standard_normal((P, head_dim)).astype(np.float32)
    m = r.uniform(-20.0, 20.0, size=P).astype(np.float32)
    l = r.uniform(0.5, 50.0, size=P).astype(np.float32)
    empty = r.random(P) < p_empty
    o[empty] = 0.0
    m[empty] = -1e30
    l[empty] = 0.0
    return dict(o=o, m=m, l=l, group_ptr=gp, groups=groups)


def kv_bytes(w) -> int:
    """K+V cache bytes a causal decode/prefill pass must read once per sequence: sum_b L_b*G*D*2*2."""
    L = w["past"].astype(np.int64) + np.diff(w["cu"]).astype(np.int64)
    return int(L.sum()) * w["G"] * w["D"] * 2 * 2
