"""Pins of the chunk-attention and merge oracle (numpy) against independent references.

- A chunk holding every key at position 0 is the C oracle's attention (pinned in
  test_oracle_attention.py) and its lse the C backward oracle's (pinned in
  test_oracle_backward.py): two separate implementations.
- Splitting the keys into chunks and merging gives the full attention: the merge
  formula, the global-position causal mask and the lse are all exercised; a wrong
  weight, sign or offset breaks the identity.
- Closed forms: a one-key chunk returns that key's value and score; rows before every
  key (causal) return o = 0, lse = -inf, which the merge treats as the identity.
"""
import numpy as np
import pytest

import oracle


def _rand(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(1, 7, 1, 1, 4), (2, 33, 4, 2, 8), (1, 50, 3, 1, 16)])
def test_full_chunk_is_attention(B, S, Hq, Hkv, D, causal):
    q, k, v = _rand(1, (B, S, Hq, D)), _rand(2, (B, S, Hkv, D)), _rand(3, (B, S, Hkv, D))
    o, lse = oracle.attention_chunk(q, k, v, causal)
    np.testing.assert_allclose(o, oracle.attention(q, k, v, causal), rtol=0, atol=1e-12)
    lse_c = oracle.attention_backward(q, k, v, np.zeros_like(q), causal)[3]
    np.testing.assert_allclose(lse, lse_c, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("cuts", [(1,), (17,), (5, 20, 21), (10, 20, 30, 40)])
def test_split_and_merge_is_attention(cuts, causal):
    """Keys cut into chunks at the given positions; each chunk at its global key
    position; merged in order = attention over all keys."""
    B, S, Hq, Hkv, D = 2, 48, 4, 2, 8
    q, k, v = _rand(11, (B, S, Hq, D)), _rand(12, (B, S, Hkv, D)), _rand(13, (B, S, Hkv, D))
    edges = [0, *cuts, S]
    o, lse = None, None
    for a, b in zip(edges[:-1], edges[1:]):
        oc, lc = oracle.attention_chunk(q, k[:, a:b], v[:, a:b], causal, q_pos0=0, k_pos0=a)
        o, lse = (oc, lc) if o is None else oracle.softmax_merge(o, lse, oc, lc)
    np.testing.assert_allclose(o, oracle.attention(q, k, v, causal), rtol=0, atol=1e-12)
    lse_c = oracle.attention_backward(q, k, v, np.zeros_like(q), causal)[3]
    np.testing.assert_allclose(lse, lse_c, rtol=0, atol=1e-12)


def test_query_block_offsets():
    """A query block at positions 30..45 against the full key range split in three:
    the block's rows see keys up to their own global position only."""
    B, S, H, D = 1, 60, 2, 8
    q, k, v = _rand(21, (B, S, H, D)), _rand(22, (B, S, H, D)), _rand(23, (B, S, H, D))
    want = oracle.attention(q, k, v, True)[:, 30:46]
    o, lse = None, None
    for a, b in ((0, 25), (25, 40), (40, 60)):
        oc, lc = oracle.attention_chunk(q[:, 30:46], k[:, a:b], v[:, a:b], True, q_pos0=30, k_pos0=a)
        o, lse = (oc, lc) if o is None else oracle.softmax_merge(o, lse, oc, lc)
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-12)


def test_one_key_chunk_closed_form():
    q, k, v = _rand(31, (1, 5, 1, 4)), _rand(32, (1, 1, 1, 4)), _rand(33, (1, 1, 1, 4))
    o, lse = oracle.attention_chunk(q, k, v, False)
    np.testing.assert_array_equal(o[0, :, 0], np.repeat(v[0, :1, 0], 5, axis=0))
    np.testing.assert_allclose(lse[0, 0], q[0, :, 0] @ k[0, 0, 0] / 2.0, rtol=0, atol=1e-15)


def test_rows_before_every_key_are_empty():
    """Causal, keys at positions 10.. and queries at 0..14: rows 0..9 see nothing."""
    q, k, v = _rand(41, (1, 15, 2, 4)), _rand(42, (1, 6, 2, 4)), _rand(43, (1, 6, 2, 4))
    o, lse = oracle.attention_chunk(q, k, v, True, q_pos0=0, k_pos0=10)
    assert np.all(o[:, :10] == 0) and np.all(np.isneginf(lse[:, :, :10]))
    assert np.all(np.isfinite(lse[:, :, 10:]))
    # row 10 sees exactly key 0 of the chunk
    np.testing.assert_array_equal(o[0, 10], v[0, 0])
    # merging with an empty result returns the other one exactly, in both orders
    o2, l2 = oracle.attention_chunk(q, k, v, False)
    for a, b in ((o, lse), (o2, l2)):
        empty_o, empty_l = np.zeros_like(a), np.full_like(b, -np.inf)
        for mo, ml in (oracle.softmax_merge(a, b, empty_o, empty_l), oracle.softmax_merge(empty_o, empty_l, a, b)):
            np.testing.assert_array_equal(mo, a)
            np.testing.assert_array_equal(ml, b)


def test_merge_symmetric_and_associative():
    g = np.random.default_rng(51)
    os_ = [g.standard_normal((2, 9, 3, 4)) for _ in range(3)]
    ls = [g.standard_normal((2, 3, 9)) * 3 for _ in range(3)]
    ab, lab = oracle.softmax_merge(os_[0], ls[0], os_[1], ls[1])
    ba, lba = oracle.softmax_merge(os_[1], ls[1], os_[0], ls[0])
    np.testing.assert_allclose(ab, ba, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lab, lba, rtol=0, atol=1e-14)
    left = oracle.softmax_merge(ab, lab, os_[2], ls[2])
    bc, lbc = oracle.softmax_merge(os_[1], ls[1], os_[2], ls[2])
    right = oracle.softmax_merge(os_[0], ls[0], bc, lbc)
    np.testing.assert_allclose(left[0], right[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(left[1], right[1], rtol=0, atol=1e-13)
    # lse of the union is log(sum exp): checked against a direct evaluation
    np.testing.assert_allclose(lab, np.log(np.exp(ls[0]) + np.exp(ls[1])), rtol=0, atol=1e-13)


def test_bf16_inputs_decode_exactly():
    g = np.random.default_rng(61)
    x = g.standard_normal((1, 6, 1, 8)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncated to bf16
    dec = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    o1, l1 = oracle.attention_chunk(bits, bits, bits, True, bf16=True)
    o2, l2 = oracle.attention_chunk(dec, dec, dec, True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# --- gradients of one chunk visit (oracle.attention_chunk_backward) --------------------

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(1, 9, 1, 1, 4), (2, 31, 4, 2, 8)])
def test_chunk_backward_whole_sequence_is_attention_backward(B, S, Hq, Hkv, D, causal):
    """One visit holding every key, with its own output and lse: the C oracle's
    attention gradients (a separate implementation, pinned by finite differences)."""
    q, k, v, g = (_rand(s, sh) for s, sh in ((21, (B, S, Hq, D)), (22, (B, S, Hkv, D)),
                                              (23, (B, S, Hkv, D)), (24, (B, S, Hq, D))))
    dq, dk, dv, lse = oracle.attention_backward(q, k, v, g, causal)
    o = oracle.attention(q, k, v, causal)
    cq, ck, cv = oracle.attention_chunk_backward(q, k, v, g, o, lse, causal)
    for a, b in ((cq, dq), (ck, dk), (cv, dv)):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_chunk_backward_visits_sum_to_attention_backward(causal):
    """Keys in three chunks at their global positions and a query block at an offset
    (rows 20..47 of the sequence): with the merged output and lse, the dq
    contributions add up to the block's rows of the full dq, and each chunk's dk, dv
    are the full dk, dv of its keys restricted to this query block -- checked by
    running the full gradients with dout zero outside the block."""
    B, S, Hq, Hkv, D = 2, 48, 4, 2, 8
    q, k, v = _rand(31, (B, S, Hq, D)), _rand(32, (B, S, Hkv, D)), _rand(33, (B, S, Hkv, D))
    g = _rand(34, (B, S, Hq, D))
    r0, r1 = 20, 48
    g[:, :r0] = 0.0  # only the query block's rows carry an output gradient
    dq, dk, dv, lse = oracle.attention_backward(q, k, v, g, causal)
    o = oracle.attention(q, k, v, causal)
    qb, gb, ob, lb = q[:, r0:r1], g[:, r0:r1], o[:, r0:r1], lse[:, :, r0:r1]
    sq = np.zeros_like(qb)
    for a, b in ((0, 13), (13, 30), (30, 48)):
        cq, ck, cv = oracle.attention_chunk_backward(qb, k[:, a:b], v[:, a:b], gb, ob, lb, causal,
                                                     q_pos0=r0, k_pos0=a)
        sq += cq
        np.testing.assert_allclose(ck, dk[:, a:b], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(cv, dv[:, a:b], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sq, dq[:, r0:r1], rtol=1e-10, atol=1e-12)


def test_chunk_backward_finite_differences_at_an_offset():
    """Central differences of L = sum(dout * o) for one visit at query position 3 and
    key position 0 (causal: rows see a shifted triangle), o and lse the visit's own."""
    B, Sq, Skv, Hq, Hkv, D, qp, kp = 1, 5, 7, 2, 1, 4, 3, 0
    q, k, v = _rand(41, (B, Sq, Hq, D)), _rand(42, (B, Skv, Hkv, D)), _rand(43, (B, Skv, Hkv, D))
    g = _rand(44, (B, Sq, Hq, D))
    o, lse = oracle.attention_chunk(q, k, v, True, qp, kp)
    dq, dk, dv = oracle.attention_chunk_backward(q, k, v, g, o, lse, True, qp, kp)

    def loss(q_, k_, v_):
        return float((g * oracle.attention_chunk(q_, k_, v_, True, qp, kp)[0]).sum())

    h = 1e-6
    for x, grad, name in ((q, dq, "q"), (k, dk, "k"), (v, dv, "v")):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)
