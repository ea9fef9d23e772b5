"""Tolerances and comparison helpers for GPU-vs-oracle parity.

Bars (stated for this path): the append without rotary is bit-exact; rotary keys are within
1e-3 absolute; fp16 attention outputs are within 2e-3 absolute + 1e-2 relative; the fp32
block-sparse path is within 1e-4: partial maxima absolute; partial o and l, and merged outputs,
within 1e-4 * max(1, |reference|) (absolute below magnitude 1; above it fp32's own rounding
grows with the magnitude, as for the unnormalised partial sums). On inputs whose sums cancel
(outlier channels), o and merged outputs are held to 1e-4 of the magnitude of their terms.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ATT_ABS, ATT_REL = 2e-3, 1e-2
ROT_ABS = 1e-3
SPARSE_TOL = 1e-4


def as_np(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x)


def assert_bits_equal(got, ref, what=""):
    g = as_np(got).view(np.uint16) if as_np(got).dtype == np.float16 else as_np(got)
    r = as_np(ref).view(np.uint16) if as_np(ref).dtype == np.float16 else as_np(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    bad = np.nonzero(g != r)
    assert bad[0].size == 0, f"{what}: {bad[0].size} elements differ, first at {[b[0] for b in bad]}"


def assert_attention_close(got, ref, what=""):
    g = as_np(got).astype(np.float64)
    r = as_np(ref).astype(np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - r)
    tol = ATT_ABS + ATT_REL * np.abs(r)
    worst = np.argmax(err - tol)
    assert np.all(err <= tol), (f"{what}: max err {err.max():.3e}, worst {g.flat[worst]} vs "
                                f"{r.flat[worst]} at {np.unravel_index(worst, g.shape)}")


def _scale(r, terms):
    """max(1, |ref|), or max(1, |ref|, terms) when the magnitude of the summed terms is given."""
    s = np.maximum(1.0, np.abs(r))
    return s if terms is None else np.maximum(s, np.abs(as_np(terms).astype(np.float64)))


def assert_sparse_partials_close(got, ref, what="", o_terms=None):
    """o_terms (optional): the magnitude of the terms summed into each partial o, sum_t p_t |v_t|
    (the oracle's o over |V|). A sum whose terms cancel carries fp32 rounding relative to its
    terms, not to its value, so with outlier channels the bar for o is taken relative to them."""
    go, gm, gl = (as_np(x).astype(np.float64) for x in got)
    ro, rm, rl = (as_np(x).astype(np.float64) for x in ref)
    assert np.all(np.abs(gm - rm) <= SPARSE_TOL), f"{what}: m max err {np.abs(gm - rm).max()}"
    assert np.all(np.abs(gl - rl) <= SPARSE_TOL * np.maximum(1.0, np.abs(rl))), \
        f"{what}: l max err {np.abs(gl - rl).max()}"
    err = np.abs(go - ro) / _scale(ro, o_terms)
    assert np.all(err <= SPARSE_TOL), f"{what}: o max scaled err {err.max():.3e}"


def assert_sparse_out_close(got, ref, what="", terms=None):
    """terms (optional): the magnitude of each merged output's terms, sum w |v| / sum w."""
    g = as_np(got).astype(np.float64)
    r = as_np(ref).astype(np.float64)
    err = np.abs(g - r) / _scale(r, terms)
    assert np.all(err <= SPARSE_TOL), f"{what}: max scaled err {err.max():.3e}"


def rows_as_decode(w, rows):
    """A workload whose sequence k is row rows[k] of w as a one-token decode: past = that row's
    position, same block-table row, same query row. For causal attention the row sees exactly
    the same keys, so the oracle can check sampled rows of a large prefill at its own cost."""
    rows = np.asarray(rows)
    seq = np.searchsorted(w["cu"], rows, side="right") - 1
    pos = w["past"][seq] + (rows - w["cu"][seq])
    sub = dict(w)
    sub["B"] = sub["T"] = len(rows)
    sub["past"] = pos.astype(np.int32)
    sub["cu"] = np.arange(len(rows) + 1, dtype=np.int32)
    sub["block_table"] = w["block_table"][seq]
    sub["query"] = w["query"][rows]
    sub["key"] = sub["value"] = sub["slot_mapping"] = None
    return sub


def host_threads():
    """Host threads for oracle runs: the cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_rows(oracle, w, kc, vc, rows=None):
    """The oracle's attention output of the given rows (every row when None) of causal paged
    workload w, as fp16 [len(rows), H*D]. Each row is computed as the equivalent one-token decode
    (rows_as_decode); the rows are dealt round-robin into chunks run on host threads (the oracle
    runs in C, outside the interpreter lock), so long and short rows spread evenly."""
    assert w["causal"] == 1, "rows_as_decode is exact only for causal attention"
    rows = np.arange(w["T"]) if rows is None else np.asarray(rows)
    n = host_threads()
    nchunks = max(1, min(len(rows), 4 * n))
    idx = [np.arange(k, len(rows), nchunks) for k in range(nchunks)]
    out = np.empty((len(rows), w["H"] * w["D"]), dtype=np.float16)
    with ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(lambda ix: oracle.paged_attention(rows_as_decode(w, rows[ix]), kc, vc),
                            idx))
    for ix, part in zip(idx, parts):
        out[ix] = part
    return out


def oracle_sparse_full(oracle, sw, q_pos=None, sample_edges=()):
    """The oracle's merged output of every (q, h) group of sparse workload sw (float32
    [Tq*hq, D]) and its partials of sample_edges (rows e*qhead + qh, in sample order). Groups are
    cut into contiguous ranges run on host threads; each range's partials are merged at once and
    dropped, so only the sample's partials are kept."""
    q, D = sw["qhead"], sw["D"]
    gp = sw["group_ptr"]
    G = len(gp) - 1
    sample = np.asarray(sample_edges, dtype=np.int64)
    n = host_threads()
    bounds = np.linspace(0, G, 4 * n + 1).astype(np.int64)

    def part(k):
        g0, g1 = int(bounds[k]), int(bounds[k + 1])
        e0, e1 = int(gp[g0]), int(gp[g1])
        o, m, l = oracle.sparse_forward(sw, edge_meta=sw["edge_meta"][e0:e1], q_pos=q_pos)
        merged = oracle.split_combine(o, m, l, lanes=q, head_dim=D,
                                      group_ptr=(gp[g0:g1 + 1] - e0).astype(np.int32),
                                      out_dtype=np.float32)
        sel = np.nonzero((sample >= e0) & (sample < e1))[0]
        prow = ((sample[sel] - e0)[:, None] * q + np.arange(q)[None, :]).reshape(-1)
        return merged, sel, o[prow], m[prow], l[prow]

    with ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(part, range(len(bounds) - 1)))
    merged = np.concatenate([p[0] for p in parts])
    po = np.empty((len(sample) * q, D), dtype=np.float32)
    pm = np.empty(len(sample) * q, dtype=np.float32)
    pl = np.empty(len(sample) * q, dtype=np.float32)
    for _, sel, o, m, l in parts:
        rows = (sel[:, None] * q + np.arange(q)[None, :]).reshape(-1)
        po[rows], pm[rows], pl[rows] = o, m, l
    return merged, (po, pm, pl)
