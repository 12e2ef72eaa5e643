"""Where the kernels' lazily moved softmax reference must move (test helper).

The decode and several-token kernels keep a running reference max m per
(query token, head) and move it only when a block's (or a 32-row step's)
largest score exceeds m by more than 8 log2 units; the accumulator and the sum
are then rescaled by 2^(m - m_new).  Whether a given input exercises that
rescale with a finite m (not the first block a wave sees) depends on the
scores and on how the rows are cut among waves.  This module replays that cut
on the host from the stored values and counts such events, so a test can
assert that its inputs really reach the branch.  It computes no attention
output.
"""
from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634
THRESHOLD = 8.0


def log2_scores(st, wl, q64, q_rows, b, layer=0):
    """[len(q_rows), Hq, n_b] scores * scale * log2 e of sequence b from the
    oracle store's stored (dequantised) keys."""
    k, _ = st.gather(b, layer)                          # [n, Hkv, D]
    G = wl.num_heads // wl.num_kv_heads
    kk = np.repeat(k, G, axis=1)                        # [n, Hq, D]
    q = q64[q_rows]                                     # [r, Hq, D]
    return np.einsum("rhd,nhd->rhn", q, kk) * (wl.scale * LOG2E)


def decode_chunks(attend_lens, W):
    """The decode's even split: the batch's blocks in one list cut into
    min(W, total) runs.  Returns [(b, first block, end block)] per run piece."""
    nb = [(int(n) + 15) // 16 for n in attend_lens]
    start = np.concatenate([[0], np.cumsum(nb)])
    total = int(start[-1])
    W = max(1, min(W, total))
    out = []
    for w in range(W):
        x0, x1 = -(-w * total // W), -(-(w + 1) * total // W)
        for b in range(len(nb)):
            a, e = max(x0, start[b]), min(x1, start[b + 1])
            if a < e:
                out.append((b, int(a - start[b]), int(e - start[b])))
    return out


def _walk(s, n_rows, r0, r1, step):
    """Finite moves of the reference over rows [r0, r1) of one score row s,
    `step` rows at a time from r0; rows >= n_rows are not seen."""
    m, grows = -np.inf, 0
    for a in range(r0, min(r1, n_rows), step):
        bm = s[a:min(a + step, n_rows)].max()
        if bm > m + THRESHOLD:
            if np.isfinite(m) and bm > m + THRESHOLD + 0.05:
                grows += 1
            m = bm
    return grows


def decode_grows(st, wl, q64, W):
    """Finite reference moves of the decode over the whole batch for W waves
    per KV head."""
    total = 0
    n = wl.attend_lens
    scores = {b: log2_scores(st, wl, q64, [b], b)[0] for b in range(wl.batch)}
    for b, j0, j1 in decode_chunks(n, W):
        s = scores[b]
        for h in range(wl.num_heads):
            total += _walk(s[h], int(n[b]), 16 * j0, 16 * j1, 16)
    return total


def extend_grows(st, wl, q64, step):
    """Finite reference moves of several-token attention, every sequence's rows
    walked from row 0 `step` rows at a time by each (query token, head)."""
    total = 0
    qls = wl.q_lens
    q0 = np.concatenate([[0], np.cumsum(qls)])
    for b in range(wl.batch):
        n, ql = int(wl.attend_lens[b]), int(qls[b])
        if ql == 0:
            continue
        s = log2_scores(st, wl, q64, list(range(q0[b], q0[b + 1])), b)
        for i in range(ql):
            seen = n - ql + i + 1
            for h in range(wl.num_heads):
                total += _walk(s[i, h], seen, 0, seen, step)
    return total
