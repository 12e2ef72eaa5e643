"""Pins for the fp64 attention oracle (CPU only).

Each pin ties the oracle to something other than itself: the pages' worked
example (inputs printed on "大模型推理加速——KV Cache篇" §2.1), closed forms,
brute-force full recomputation, and torch's own scaled_dot_product_attention
and softmax run in fp64 on the CPU (independent library routines).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


@pytest.fixture
def worked(golden_dir):
    g = _load(golden_dir, "worked_example.json")
    X1, X2 = np.array(g["X_step1"]), np.array(g["X_step2"])
    WQ, WK, WV = np.array(g["W_Q"]), np.array(g["W_K"]), np.array(g["W_V"])
    return dict(g=g, X1=X1, X2=X2, WQ=WQ, WK=WK, WV=WV, scale=1.0 / g["score_divisor"])


def test_worked_example_first_row_is_first_value(worked):
    # Closed form: a query that sees a single key returns that key's value row.
    X2, WQ, WK, WV = worked["X2"], worked["WQ"], worked["WK"], worked["WV"]
    Q, K, V = X2 @ WQ, X2 @ WK, X2 @ WV
    out = attention.decode_attention(Q[:1], K[:1, None, :], V[:1, None, :], worked["scale"])
    assert np.array_equal(out[0], V[0])
    full = attention.causal_attention(Q, K, V, worked["scale"])
    assert np.array_equal(full[0], V[0])


def test_worked_example_matches_page_procedure_in_torch(worked):
    # The page's own procedure (scores / 2 + printed mask, F.softmax, matmul),
    # evaluated by torch in fp64, against the oracle's causal and decode forms.
    g = worked["g"]
    for X, mask in ((worked["X1"], g["mask_step1"]), (worked["X2"], g["mask_step2"])):
        Xt = torch.tensor(X, dtype=torch.float64)
        Q = Xt @ torch.tensor(g["W_Q"], dtype=torch.float64)
        K = Xt @ torch.tensor(g["W_K"], dtype=torch.float64)
        V = Xt @ torch.tensor(g["W_V"], dtype=torch.float64)
        m = torch.tensor([[float(x) for x in row] for row in mask], dtype=torch.float64)
        ref = F.softmax(Q @ K.T / g["score_divisor"] + m, dim=-1) @ V
        ours = attention.causal_attention(Q.numpy(), K.numpy(), V.numpy(), worked["scale"])
        np.testing.assert_allclose(ours, ref.numpy(), rtol=0, atol=1e-15)
        # every row i is also a decode step over keys 0..i
        for i in range(X.shape[0]):
            dec = attention.decode_attention(Q[i:i + 1].numpy(), K[:i + 1, None].numpy(),
                                             V[:i + 1, None].numpy(), worked["scale"])
            np.testing.assert_allclose(dec[0], ref[i].numpy(), rtol=0, atol=1e-15)


def test_worked_example_cache_reuse(worked):
    # Step 1 rows equal step 2's first two rows (history does not change when a
    # token is appended), and the cached decode of the third token equals the
    # full recomputation's last row (the page's claim in §2.2).
    X1, X2, WQ, WK, WV, s = (worked[k] for k in ("X1", "X2", "WQ", "WK", "WV", "scale"))
    full1 = attention.causal_attention(X1 @ WQ, X1 @ WK, X1 @ WV, s)
    full2 = attention.causal_attention(X2 @ WQ, X2 @ WK, X2 @ WV, s)
    np.testing.assert_allclose(full1, full2[:2], rtol=0, atol=1e-16)
    K_cached, V_cached = X1 @ WK, X1 @ WV                   # K_last, V_last
    x_new = X2[2:3]
    K_all = np.concatenate([K_cached, x_new @ WK])[:, None, :]
    V_all = np.concatenate([V_cached, x_new @ WV])[:, None, :]
    dec = attention.decode_attention(x_new @ WQ, K_all, V_all, s)
    np.testing.assert_allclose(dec[0], full2[2], rtol=0, atol=1e-16)


@pytest.mark.parametrize("hq,hkv,d,n", [(1, 1, 4, 1), (4, 4, 8, 9), (8, 2, 64, 33), (8, 1, 16, 17),
                                        (6, 3, 8, 40), (16, 2, 128, 64)])
def test_decode_equals_last_row_of_full_recompute(hq, hkv, d, n):
    rng = np.random.default_rng(hq * 1000 + n)
    Q = rng.standard_normal((n, hq, d))
    K = rng.standard_normal((n, hkv, d))
    V = rng.standard_normal((n, hkv, d))
    s = 1.0 / math.sqrt(d)
    dec = attention.decode_attention(Q[-1], K, V, s)
    G = hq // hkv
    for h in range(hq):
        full = attention.causal_attention(Q[:, h], K[:, h // G], V[:, h // G], s)
        np.testing.assert_allclose(dec[h], full[-1], rtol=1e-12, atol=1e-14)


def _sdpa_reference(q, K, V, scale):
    # torch's SDPA in fp64 on the CPU; enable_gqa groups query heads contiguously.
    qt = torch.tensor(q, dtype=torch.float64)[None, :, None, :]          # [1, Hq, 1, D]
    kt = torch.tensor(K, dtype=torch.float64).permute(1, 0, 2)[None]      # [1, Hkv, n, D]
    vt = torch.tensor(V, dtype=torch.float64).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(), scale=scale,
                                       enable_gqa=True)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (8, 1), (64, 8), (32, 8)])
def test_decode_matches_torch_sdpa_fp64(hq, hkv):
    rng = np.random.default_rng(hq + 7 * hkv)
    d, n = 128, 50
    q = rng.standard_normal((hq, d))
    K = rng.standard_normal((n, hkv, d))
    V = rng.standard_normal((n, hkv, d))
    s = float(np.float32(1 / math.sqrt(d)))
    np.testing.assert_allclose(attention.decode_attention(q, K, V, s), _sdpa_reference(q, K, V, s),
                               rtol=1e-12, atol=1e-13)


def test_planted_head_mapping_mistake_is_caught():
    # A plausible slip -- interleaved groups (h % Hkv) instead of contiguous
    # ones -- must fail the SDPA pin, so the pin has teeth.
    def wrong(q, K, V, scale):
        hq, hkv = q.shape[0], K.shape[1]
        out = np.empty_like(q)
        for h in range(hq):
            g = h % hkv
            sc = scale * (K[:, g] @ q[h])
            w = np.exp(sc - sc.max())
            out[h] = w @ V[:, g] / w.sum()
        return out
    rng = np.random.default_rng(5)
    q, K, V = rng.standard_normal((8, 16)), rng.standard_normal((20, 2, 16)), rng.standard_normal((20, 2, 16))
    ref = _sdpa_reference(q, K, V, 0.25)
    assert not np.allclose(wrong(q, K, V, 0.25), ref, atol=1e-6)
    assert np.allclose(attention.decode_attention(q, K, V, 0.25), ref, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(11)
    d = 64
    # single token: output is that token's value row for every head of the group
    q = rng.standard_normal((8, d))
    K = rng.standard_normal((1, 2, d))
    V = rng.standard_normal((1, 2, d))
    out = attention.decode_attention(q, K, V, 0.125)
    for h in range(8):
        assert np.array_equal(out[h], V[0, h // 4])
    # identical keys: uniform weights -> mean of the values
    n = 37
    K = np.repeat(rng.standard_normal((1, 2, d)), n, axis=0)
    V = rng.standard_normal((n, 2, d))
    out = attention.decode_attention(q, K, V, 0.125)
    for h in range(8):
        np.testing.assert_allclose(out[h], V[:, h // 4].mean(axis=0), rtol=0, atol=1e-14)
    # constant values: output is that constant whatever the scores
    K = rng.standard_normal((n, 2, d)) * 5
    V = np.broadcast_to(rng.standard_normal((1, 2, d)), (n, 2, d))
    out = attention.decode_attention(q, K, V, 0.125)
    for h in range(8):
        np.testing.assert_allclose(out[h], V[0, h // 4], rtol=1e-15, atol=1e-15)
    # scale 0: plain mean of the values
    V = rng.standard_normal((n, 2, d))
    out = attention.decode_attention(q, K, V, 0.0)
    np.testing.assert_allclose(out[0], V[:, 0].mean(axis=0), atol=1e-14)


def test_outputs_lie_in_the_convex_hull():
    rng = np.random.default_rng(3)
    q, K, V = rng.standard_normal((8, 32)) * 3, rng.standard_normal((100, 4, 32)), rng.standard_normal((100, 4, 32))
    out = attention.decode_attention(q, K, V, 1.0)
    for h in range(8):
        g = h // 2
        assert np.all(out[h] <= V[:, g].max(axis=0) + 1e-12)
        assert np.all(out[h] >= V[:, g].min(axis=0) - 1e-12)


def test_batch_wrapper_is_per_sequence():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((3, 4, 8))
    ks = [rng.standard_normal((n, 2, 8)) for n in (1, 5, 17)]
    vs = [rng.standard_normal((n, 2, 8)) for n in (1, 5, 17)]
    out = attention.decode_attention_batch(q, ks, vs, 0.3)
    for b in range(3):
        np.testing.assert_array_equal(out[b], attention.decode_attention(q[b], ks[b], vs[b], 0.3))


# -- several new tokens per sequence (verify pass / prefill chunk) ----------------

def test_extend_worked_example_against_page_procedure(worked):
    # The page's step-2 prompt of three tokens, with its printed causal mask, run
    # by torch in fp64 (the page's procedure), against the oracle's multi-token
    # form: all three tokens at once (an uncached prefill), and the last two
    # tokens as a chunk over the first one cached (a chunked prefill / verify).
    g = worked["g"]
    Xt = torch.tensor(worked["X2"], dtype=torch.float64)
    Q = Xt @ torch.tensor(g["W_Q"], dtype=torch.float64)
    K = Xt @ torch.tensor(g["W_K"], dtype=torch.float64)
    V = Xt @ torch.tensor(g["W_V"], dtype=torch.float64)
    m = torch.tensor([[float(x) for x in row] for row in g["mask_step2"]], dtype=torch.float64)
    ref = (F.softmax(Q @ K.T / g["score_divisor"] + m, dim=-1) @ V).numpy()
    Qn, Kn, Vn = Q.numpy()[:, None, :], K.numpy()[:, None, :], V.numpy()[:, None, :]
    whole = attention.extend_attention(Qn, Kn, Vn, worked["scale"])
    np.testing.assert_allclose(whole[:, 0], ref, rtol=0, atol=1e-15)
    chunk = attention.extend_attention(Qn[1:], Kn, Vn, worked["scale"])
    np.testing.assert_allclose(chunk[:, 0], ref[1:], rtol=0, atol=1e-15)
    # first row is the first value row exactly (it sees one key)
    assert np.array_equal(whole[0, 0], Vn[0, 0])


def test_extend_of_one_token_is_decode():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((1, 8, 32))
    K, V = rng.standard_normal((19, 2, 32)), rng.standard_normal((19, 2, 32))
    np.testing.assert_array_equal(attention.extend_attention(q, K, V, 0.2)[0],
                                  attention.decode_attention(q[0], K, V, 0.2))


def _sdpa_causal(q, K, V, scale):
    # torch SDPA in fp64 with an explicit boolean mask: query i (of nq) sees key
    # j iff j <= i + n - nq; enable_gqa groups query heads contiguously.
    nq, n = q.shape[0], K.shape[0]
    mask = torch.ones(nq, n, dtype=torch.bool).tril(diagonal=n - nq)
    qt = torch.tensor(q, dtype=torch.float64).permute(1, 0, 2)[None]      # [1, Hq, nq, D]
    kt = torch.tensor(K, dtype=torch.float64).permute(1, 0, 2)[None]      # [1, Hkv, n, D]
    vt = torch.tensor(V, dtype=torch.float64).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(), attn_mask=mask, scale=scale,
                                       enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,nq,n", [(8, 2, 5, 40), (4, 4, 16, 16), (16, 1, 3, 70), (6, 3, 9, 9),
                                         (64, 8, 2, 33)])
def test_extend_matches_torch_sdpa_with_causal_mask(hq, hkv, nq, n):
    rng = np.random.default_rng(hq * 31 + nq)
    d = 64
    q = rng.standard_normal((nq, hq, d))
    K, V = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    s = float(np.float32(1 / math.sqrt(d)))
    np.testing.assert_allclose(attention.extend_attention(q, K, V, s), _sdpa_causal(q, K, V, s),
                               rtol=1e-12, atol=1e-13)


def test_extend_equals_last_rows_of_full_recompute():
    rng = np.random.default_rng(8)
    hq, hkv, d, n, nq = 6, 2, 16, 23, 7
    Q = rng.standard_normal((n, hq, d))
    K, V = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    ext = attention.extend_attention(Q[n - nq:], K, V, 0.25)
    for h in range(hq):
        full = attention.causal_attention(Q[:, h], K[:, h // 3], V[:, h // 3], 0.25)
        np.testing.assert_allclose(ext[:, h], full[n - nq:], rtol=1e-12, atol=1e-14)


def test_chunked_prefill_equals_one_pass():
    # A prompt processed in chunks (each chunk attending to everything before
    # it) gives the same rows as processing it whole.
    rng = np.random.default_rng(12)
    n, hq, hkv, d = 30, 4, 2, 8
    Q = rng.standard_normal((n, hq, d))
    K, V = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    whole = attention.extend_attention(Q, K, V, 0.3)
    start = 0
    for c in (7, 1, 16, 6):
        part = attention.extend_attention(Q[start:start + c], K[:start + c], V[:start + c], 0.3)
        np.testing.assert_allclose(part, whole[start:start + c], rtol=1e-13, atol=1e-15)
        start += c


def test_planted_causal_offset_mistake_is_caught():
    # Off by one in the visible range (the token not seeing itself) must fail
    # the SDPA pin.
    def wrong(q, K, V, scale):
        nq, hq, d = q.shape
        n, hkv, _ = K.shape
        out = np.empty_like(q)
        for i in range(nq):
            vis = max(1, n - nq + i)
            for h in range(hq):
                sc = scale * (K[:vis, h // (hq // hkv)] @ q[i, h])
                w = np.exp(sc - sc.max())
                out[i, h] = w @ V[:vis, h // (hq // hkv)] / w.sum()
        return out
    rng = np.random.default_rng(2)
    q, K, V = rng.standard_normal((4, 4, 8)), rng.standard_normal((10, 2, 8)), rng.standard_normal((10, 2, 8))
    ref = _sdpa_causal(q, K, V, 0.4)
    assert not np.allclose(wrong(q, K, V, 0.4), ref, atol=1e-6)
    assert np.allclose(attention.extend_attention(q, K, V, 0.4), ref, atol=1e-12)


# -- sliding window ---------------------------------------------------------------

def _sdpa_window(q, K, V, scale, window):
    # torch SDPA in fp64 with a banded boolean mask: query i (position
    # p = n - nq + i) sees key j iff p - window < j <= p.
    nq, n = q.shape[0], K.shape[0]
    causal = torch.ones(nq, n, dtype=torch.bool).tril(diagonal=n - nq)
    band = torch.ones(nq, n, dtype=torch.bool).triu(diagonal=n - nq - window + 1)
    qt = torch.tensor(q, dtype=torch.float64).permute(1, 0, 2)[None]
    kt = torch.tensor(K, dtype=torch.float64).permute(1, 0, 2)[None]
    vt = torch.tensor(V, dtype=torch.float64).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(), attn_mask=causal & band, scale=scale,
                                       enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,nq,n,window", [(8, 2, 1, 40, 7), (8, 2, 5, 40, 16), (4, 4, 16, 16, 3),
                                                (16, 1, 3, 70, 64), (6, 3, 9, 30, 1)])
def test_window_matches_torch_sdpa_with_banded_mask(hq, hkv, nq, n, window):
    rng = np.random.default_rng(hq * 13 + window)
    d = 32
    q = rng.standard_normal((nq, hq, d))
    K, V = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    np.testing.assert_allclose(attention.extend_attention(q, K, V, 0.2, window=window),
                               _sdpa_window(q, K, V, 0.2, window), rtol=1e-12, atol=1e-13)


def test_window_special_cases():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 4, 16))
    K, V = rng.standard_normal((25, 2, 16)), rng.standard_normal((25, 2, 16))
    full = attention.extend_attention(q, K, V, 0.3)
    # a window at least as long as the history changes nothing
    for w in (25, 26, 1000):
        np.testing.assert_array_equal(attention.extend_attention(q, K, V, 0.3, window=w), full)
    # a window of one row: each token returns its own value row
    one = attention.extend_attention(q, K, V, 0.3, window=1)
    for i in range(3):
        for h in range(4):
            assert np.array_equal(one[i, h], V[22 + i, h // 2])
    # brute force: the window equals plain attention over the sliced history
    w = 9
    win = attention.extend_attention(q, K, V, 0.3, window=w)
    for i in range(3):
        p = 22 + i
        dec = attention.decode_attention(q[i], K[p - w + 1:p + 1], V[p - w + 1:p + 1], 0.3)
        np.testing.assert_allclose(win[i], dec, rtol=1e-13, atol=1e-15)


def test_planted_window_off_by_one_is_caught():
    def wrong(q, K, V, scale, window):
        # sees window + 1 rows
        nq, hq, d = q.shape
        n, hkv, _ = K.shape
        out = np.empty_like(q)
        for i in range(nq):
            p = n - nq + i
            lo = max(0, p - window)
            for h in range(hq):
                sc = scale * (K[lo:p + 1, h // (hq // hkv)] @ q[i, h])
                wt = np.exp(sc - sc.max())
                out[i, h] = wt @ V[lo:p + 1, h // (hq // hkv)] / wt.sum()
        return out
    rng = np.random.default_rng(6)
    q, K, V = rng.standard_normal((2, 4, 8)), rng.standard_normal((20, 2, 8)), rng.standard_normal((20, 2, 8))
    ref = _sdpa_window(q, K, V, 0.5, 5)
    assert not np.allclose(wrong(q, K, V, 0.5, 5), ref, atol=1e-6)
    assert np.allclose(attention.extend_attention(q, K, V, 0.5, window=5), ref, atol=1e-12)


# -- cascade (shared-prefix) decode -------------------------------------------

@pytest.mark.parametrize("hq,hkv,n", [(4, 1, 40), (8, 2, 300), (32, 8, 129)])
def test_cascade_decode_equals_decode(hq, hkv, n):
    # the merge of the prefix's and the own rows' partials is decode attention
    # over all rows, at every split point
    rng = np.random.default_rng(n + hq)
    q = rng.standard_normal((hq, 64))
    k = rng.standard_normal((n, hkv, 64)) * 2.0
    v = rng.standard_normal((n, hkv, 64))
    ref = attention.decode_attention(q, k, v, 0.125)
    for prefix in (1, 16, n // 2, n - 1):
        got = attention.cascade_decode_attention(q, k, v, 0.125, prefix)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), prefix


def test_cascade_split_point_matters_only_through_rows():
    # two sequences forked from one prefix: their outputs agree with a decode
    # over (shared prefix + own rows), and the prefix's rows enter both
    rng = np.random.default_rng(5)
    P, hq, hkv, d = 48, 8, 2, 32
    kp, vp = rng.standard_normal((P, hkv, d)), rng.standard_normal((P, hkv, d))
    for own in (1, 17, 100):
        ko, vo = rng.standard_normal((own, hkv, d)), rng.standard_normal((own, hkv, d))
        q = rng.standard_normal((hq, d))
        k, v = np.concatenate([kp, ko]), np.concatenate([vp, vo])
        got = attention.cascade_decode_attention(q, k, v, 0.2, P)
        assert np.allclose(got, attention.decode_attention(q, k, v, 0.2), rtol=1e-12, atol=1e-12)
        # dropping the prefix changes the answer (the prefix is really attended)
        assert not np.allclose(got, attention.decode_attention(q, ko, vo, 0.2), atol=1e-3)


def test_planted_unscaled_merge_is_caught():
    # merging the two partials without rescaling to the common max is a
    # plausible mistake; the pin against decode_attention must reject it
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 16))
    k = rng.standard_normal((60, 1, 16)) * 3.0
    v = rng.standard_normal((60, 1, 16))
    ref = attention.decode_attention(q, k, v, 0.5)
    scores = 0.5 * (k[:, 0, :] @ q[0])
    m1, l1, a1 = attention._partial(scores[:20], v[:20, 0, :])
    m2, l2, a2 = attention._partial(scores[20:], v[20:, 0, :])
    wrong = (a1 + a2) / (l1 + l2)
    assert not np.allclose(wrong, ref[0], atol=1e-3)
    assert np.allclose(attention.cascade_decode_attention(q, k, v, 0.5, 20)[0], ref[0], rtol=1e-12, atol=1e-12)


def test_cascade_rejects_a_split_outside_the_rows():
    q, k = np.zeros((2, 8)), np.zeros((5, 1, 8))
    for prefix in (0, 5, 7):
        with pytest.raises(ValueError):
            attention.cascade_decode_attention(q, k, k, 1.0, prefix)
