"""Tolerances and comparison helpers for GPU-vs-oracle parity.

Bars (stated for this path): the append without rotary is bit-exact; rotary keys are within
1e-3 absolute; fp16 attention outputs are within 2e-3 absolute + 1e-2 relative; the fp32
block-sparse path is within 1e-4 (merged outputs and partial maxima absolute, partial o and l
relative to max(1, |reference|) because they are unnormalised sums).
"""
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


def assert_sparse_partials_close(got, ref, what=""):
    go, gm, gl = (as_np(x).astype(np.float64) for x in got)
    ro, rm, rl = (as_np(x).astype(np.float64) for x in ref)
    assert np.all(np.abs(gm - rm) <= SPARSE_TOL), f"{what}: m max err {np.abs(gm - rm).max()}"
    assert np.all(np.abs(gl - rl) <= SPARSE_TOL * np.maximum(1.0, np.abs(rl))), \
        f"{what}: l max err {np.abs(gl - rl).max()}"
    assert np.all(np.abs(go - ro) <= SPARSE_TOL * np.maximum(1.0, np.abs(ro))), \
        f"{what}: o max err {np.abs(go - ro).max()}"


def assert_sparse_out_close(got, ref, what=""):
    g = as_np(got).astype(np.float64)
    r = as_np(ref).astype(np.float64)
    assert np.all(np.abs(g - r) <= SPARSE_TOL), f"{what}: max err {np.abs(g - r).max()}"


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
