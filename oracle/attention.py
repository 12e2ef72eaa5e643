"""fp64 decode attention: the plain definition, no tiling, no online softmax.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (the pages' statement of the decode step):

* One new query token per sequence attends over every cached K/V row of that
  sequence plus its own newly appended row: append first, then attend
  ("苦猿的大模型日记 · Day45 · 大模型推理加速", PART 02, the ``torch.cat`` of the new
  K/V onto the cache followed by ``attention(new_q, k_cache, v_cache)``;
  "大模型推理加速——KV Cache篇" §2.2, K_cur/V_cur concatenated onto the cached
  K_last/V_last).
* Per head, scores = q . K^T, weights = softmax(scores * scale), output =
  weights . V ("LLM推理优化实战：从KV-Cache到Continuous Batching…" §1.1
  ``attention_step``; "苦猿的大模型日记" PART 02, softmax(QK^T/sqrt(d))V).  The
  scale is passed in explicitly (the kernel's fp32 value) so both sides use the
  same number.
* GQA: the query heads are split into contiguous groups, each sharing one KV
  head, so query head h reads KV head h // (Hq / Hkv)
  ("大模型推理加速核心KV Cache 复用机制与内存布局优化" §二; "大模型推理加速——KV Cache篇"
  §6.2).  Hkv == Hq is MHA, Hkv == 1 is MQA.
* Decode needs no causal mask: with one query row at the last position every
  cached column is visible (the mask of "苦猿的大模型日记" PART 04's
  ``naive_attention`` keeps all kv_len columns for q_len = 1; the LLaMA code in
  "大模型推理加速——KV Cache篇" §3 builds a mask only when seqlen > 1).

``extend_attention`` is the same step for several new query tokens per
sequence -- the target model's parallel pass over the draft tokens of
speculative decoding ("LLM推理优化实战…" §4.2, all gamma candidates verified in
one forward pass) or one chunk of a chunked prefill ("苦猿的大模型日记" PART 03,
long-prompt prefill where q_len > 1).  The new tokens are appended first, then
each one attends causally: the token at position p sees positions 0..p, which
is the mask of "苦猿的大模型日记" PART 04's ``naive_attention`` (lower triangle
shifted by kv_len - q_len).

A sliding window (``window`` > 0) limits what each token sees to its own
row and the window - 1 rows before it ("苦猿的大模型日记" PART 02: the sliding
window or KV eviction trades visible history for a fixed cache bound;
"LLM推理优化实战…" §7.2 names sliding-window attention among the forms that
restrict the attention range).  The pages give no formula; the plainest
reading, taken here, is that the token at position p sees positions
max(0, p - window + 1) .. p.

``cascade_decode_attention`` is decode attention taken apart at a fork point:
when many sequences share one prefix (requests under one system prompt share
its physical blocks, "大模型推理加速核心KV Cache 复用机制与内存布局优化" §三;
"苦猿的大模型日记" PART 02 reuses identical prefixes across requests), the
prefix rows and each sequence's own rows are attended apart, each giving a
running max, sum and weighted value sum, and the two are combined with the
merge of partial softmax results ("大模型推理加速核心KV Cache 复用机制与内存布局
优化" §四, merging between blocks; the recurrence of "LLM推理优化实战…" §3.2).
Exactly (up to rounding) the same as ``decode_attention`` over all rows.

``causal_attention`` is the full-recompute definition (page 5's
``naive_attention`` with ``tril(diagonal = kv_len - q_len)``), written here
without torch, used to pin ``decode_attention`` by brute force.
"""
from __future__ import annotations

import numpy as np


def decode_attention(q, k, v, scale):
    """Decode attention of one query token over a contiguous history.

    q: [Hq, D]   query of the new token (any real dtype; upcast to fp64)
    k, v: [n, Hkv, D]  the sequence's K/V rows in position order, the newly
        appended token last (n >= 1)
    scale: float, the softmax scale (e.g. fp32(1/sqrt(D)))
    returns: [Hq, D] fp64
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, d = q.shape
    n, hkv, dk = k.shape
    if n < 1:
        raise ValueError("decode attention needs at least one key (the new token)")
    if dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if hq % hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    scale = float(scale)
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        scores = scale * (k[:, g, :] @ q[h])          # [n]
        w = np.exp(scores - scores.max())             # softmax numerator
        out[h] = (w @ v[:, g, :]) / w.sum()
    return out


def decode_attention_batch(q, k_list, v_list, scale):
    """Apply ``decode_attention`` sequence by sequence.

    q: [B, Hq, D]; k_list[b], v_list[b]: [n_b, Hkv, D].  Returns [B, Hq, D].
    """
    q = np.asarray(q)
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(q.shape[0]):
        out[b] = decode_attention(q[b], k_list[b], v_list[b], scale)
    return out


def _partial(scores, v):
    """(max, sum of exp(s - max), sum of exp(s - max) * v) of one row range."""
    m = scores.max()
    w = np.exp(scores - m)
    return m, w.sum(), w @ v


def cascade_decode_attention(q, k, v, scale, prefix):
    """Decode attention of one query token, the rows split at ``prefix``.

    q: [Hq, D]; k, v: [n, Hkv, D] as for ``decode_attention``; 0 < prefix < n.
    Rows [0, prefix) (the shared prefix) and [prefix, n) (the sequence's own
    rows) each give a partial (m, l, acc); the output is
    (acc_1 e^(m_1 - M) + acc_2 e^(m_2 - M)) / (l_1 e^(m_1 - M) + l_2 e^(m_2 - M)),
    M = max(m_1, m_2).  returns: [Hq, D] fp64
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, d = q.shape
    n, hkv, _ = k.shape
    if not 0 < prefix < n:
        raise ValueError("need 0 < prefix < n")
    if hq % hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        scores = float(scale) * (k[:, g, :] @ q[h])
        m1, l1, a1 = _partial(scores[:prefix], v[:prefix, g, :])
        m2, l2, a2 = _partial(scores[prefix:], v[prefix:, g, :])
        big = max(m1, m2)
        c1, c2 = np.exp(m1 - big), np.exp(m2 - big)
        out[h] = (a1 * c1 + a2 * c2) / (l1 * c1 + l2 * c2)
    return out


def extend_attention(q, k, v, scale, window=0):
    """Attention of the last nq tokens of a sequence over its whole history.

    q: [nq, Hq, D]   queries of the nq newest tokens, oldest first
    k, v: [n, Hkv, D]  the sequence's K/V rows in position order, the nq new
        tokens' rows last (n >= nq >= 1)
    scale: float, the softmax scale
    window: 0 for none, else each token sees at most this many rows ending at
        its own
    returns: [nq, Hq, D] fp64; row i is the token at position p = n - nq + i,
        which attends over rows max(0, p - window + 1) .. p (0 .. p without a
        window).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, hq, d = q.shape
    n, hkv, dk = k.shape
    if not 1 <= nq <= n:
        raise ValueError("need 1 <= nq <= n")
    if dk != d or v.shape != k.shape or hq % hkv != 0:
        raise ValueError("shape mismatch")
    if window < 0:
        raise ValueError("window must be >= 0")
    group = hq // hkv
    scale = float(scale)
    out = np.empty((nq, hq, d), dtype=np.float64)
    for i in range(nq):
        p = n - nq + i                                # this token's position
        first = max(0, p - window + 1) if window else 0
        for h in range(hq):
            g = h // group
            scores = scale * (k[first:p + 1, g, :] @ q[i, h])
            w = np.exp(scores - scores.max())
            out[i, h] = (w @ v[first:p + 1, g, :]) / w.sum()
    return out


def causal_attention(q, k, v, scale):
    """Full causal attention for one head: q [nq, D], k/v [nk, D], nk >= nq.

    Row i may see key columns j <= i + (nk - nq) (the lower triangle shifted
    so the last query row sees every key), scores are scaled, softmax'd along
    the key axis with masked entries excluded, then multiplied by V.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    out = np.empty((nq, v.shape[1]), dtype=np.float64)
    for i in range(nq):
        visible = i + (nk - nq) + 1                    # columns 0 .. visible-1
        scores = np.array([scale * float(q[i] @ k[j]) for j in range(visible)])
        w = np.exp(scores - scores.max())
        w = w / w.sum()
        out[i] = sum(w[j] * v[j] for j in range(visible))
    return out
