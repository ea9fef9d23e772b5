"""Test-side model of the lazily raised running maximum that the prefill kernel's online softmax
uses: for each (row, head) column the keys are taken in 64-key tiles from key 0, and the running
maximum (log2 units) is raised only when a tile's maximum exceeds it by more than 8; O and l are
rescaled by 2^(m_old - m_new) exactly then. The final O / l equals softmax attention up to
rounding, whatever the slack.

raise_columns counts the columns whose maximum is raised after their first tile, i.e. where the
kernel's rescale branch runs; lazy_attention replays the scheme in float64, optionally with a
planted mistake in the rescale, to show that the test inputs can tell the mistakes apart.
Nothing here is imported by the library or the oracle.
"""
import numpy as np

TILE, SLACK = 64, 8.0

# Paged workloads whose keys grow by x3-x4 past a position (key_step), so the scores of most
# prefill columns rise by more than 2^8 after their first 64-key tile: Q 1, 4, 16; D 64, 128;
# causal and not; one case with two raises per column.
RAISE_CASES = [
    dict(seed=180, past=[100], n_new=[90], num_heads=4, kv_num_heads=4, head_size=64,
         block_size=16, key_step=[(64, 4.0)]),
    dict(seed=181, past=[64, 200], n_new=[40, 64], num_heads=32, kv_num_heads=8,
         head_size=128, block_size=32, key_step=[(64, 4.0)]),
    dict(seed=182, past=[150], n_new=[24], num_heads=32, kv_num_heads=2, head_size=128,
         block_size=16, causal=0, key_step=[(128, 4.0)]),
    dict(seed=183, past=[300, 90], n_new=[50, 33], num_heads=16, kv_num_heads=4,
         head_size=64, block_size=16, causal=0, packed=True, key_step=[(64, 3.0), (192, 2.0)]),
    dict(seed=184, past=[80], n_new=[129], num_heads=8, kv_num_heads=8, head_size=128,
         block_size=16, key_step=[(64, 4.0)]),
    dict(seed=185, past=[500], n_new=[40], num_heads=32, kv_num_heads=2, head_size=64,
         block_size=32, key_step=[(256, 4.0)]),
]


def _columns(w, kc, vc=None):
    """Per prefill-path row: (row index, scores [H, lim] in log2 units, V rows [lim, H, D])."""
    H, G, D, bs = w["H"], w["G"], w["D"], w["bs"]
    Q = H // G
    ncb = 1 if Q <= 16 else (2 if Q <= 32 else 4)
    q = w["query"][:, :H * D].astype(np.float64).reshape(w["T"], H, D)
    for b in range(w["B"]):
        n = int(w["cu"][b + 1] - w["cu"][b])
        past = int(w["past"][b])
        L = past + n
        if n * Q <= 16 * ncb:
            continue  # decode-like sequence: its rows go to the decode kernel
        blks = w["block_table"][b, :(L + bs - 1) // bs]
        K = kc[blks].reshape(-1, G, D)[:L].astype(np.float64)
        V = vc[blks].reshape(-1, G, D)[:L].astype(np.float64) if vc is not None else None
        heads = np.arange(H) // Q
        for t in range(n):
            i = int(w["cu"][b]) + t
            lim = past + t + 1 if w["causal"] else L
            s = np.einsum("hd,jhd->hj", q[i], K[:lim, heads]) * w["scale"] / np.log(2.0)
            yield i, s, (V[:lim, heads] if V is not None else None)


def raise_columns(w, kc):
    """(columns with a raise after their first tile, prefill-path columns)."""
    raised = total = 0
    for _, s, _ in _columns(w, kc):
        for h in range(s.shape[0]):
            m, r = -np.inf, False
            for k0 in range(0, s.shape[1], TILE):
                mt = s[h, k0:k0 + TILE].max()
                if mt > m + SLACK:
                    r |= m > -np.inf
                    m = mt
            raised += r
            total += 1
    return raised, total


def lazy_attention(w, kc, vc, mistake=None):
    """Rows of the prefill path computed with the lazy maximum; returns (row indices, [R, H*D]).
    mistake: None, "no_o_rescale", "no_l_rescale" or "alpha_x2"."""
    rows, outs = [], []
    for i, s, V in _columns(w, kc, vc):
        H, D = s.shape[0], V.shape[2]
        out = np.zeros((H, D))
        for h in range(H):
            m, l, o = -np.inf, 0.0, np.zeros(D)
            for k0 in range(0, s.shape[1], TILE):
                st = s[h, k0:k0 + TILE]
                mt = st.max()
                alpha = 1.0
                if mt > m + SLACK:
                    alpha = 0.0 if m == -np.inf else 2.0 ** (m - mt)
                    if mistake == "alpha_x2":
                        alpha *= 2.0
                    m = mt
                p = 2.0 ** (st - m)
                l = (l if mistake == "no_l_rescale" else l * alpha) + p.sum()
                o = (o if mistake == "no_o_rescale" else o * alpha) + p @ V[k0:k0 + TILE, h]
            out[h] = o / l
        rows.append(i)
        outs.append(out.reshape(-1))
    return np.array(rows), np.array(outs)
