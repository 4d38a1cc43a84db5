"""Pins of the CPU oracle's layout change against what the pages fix.

The seq->head exchange: "Sequence Parallelism II: DeepSpeed Ulysses and
All-to-All Attention" sections 1 and 3, and "Comparing Ulysses and Megatron
Sequence Parallelism" sections "DeepSpeed Attention" / "DeepSpeed Attention
costs".  None of these checks re-types the oracle's index formula: they use
the page's worked example, numpy slicing of a global tensor (what "all heads
for my tokens" and "all tokens for my heads" mean), bijection and inverse
identities, and the printed traffic numbers.
"""
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle


def _parse_kv(path):
    out = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            key, val = line.split(None, 1)
            out[key] = val
    return out


def _global_to_seq(X, P):
    """Sequence partition: rank i owns contiguous tokens [i*S/P, (i+1)*S/P)."""
    return np.stack(np.split(X, P, axis=1))


def _global_to_head(X, P):
    """Head partition: rank j owns contiguous heads [j*H/P, (j+1)*H/P), all tokens."""
    return np.stack(np.split(X, P, axis=2))


def test_worked_rank_map(golden_dir):
    """Page 1's listing: rank 0 holds S0H0..S0H3 before, S0H0,S1H0,S2H0,S3H0 after."""
    lines = open(os.path.join(golden_dir, "worked_rank_map.txt")).read()
    P = int(re.search(r"^ranks (\d+)", lines, re.M).group(1))
    H = int(re.search(r"^heads (\d+)", lines, re.M).group(1))
    before = re.search(r"^before 0: (.*)$", lines, re.M).group(1).split()
    after = re.search(r"^after 0: (.*)$", lines, re.M).group(1).split()

    # The tiny workload's shape: 256 tokens, head_dim 32, one batch.
    S, D, B = 256, 32, 1
    Sp = S // P
    # Tag every element with (sequence shard k, head h): value 1000*k + h.
    X = np.empty((B, S, H, D), dtype=np.int32)
    for k in range(P):
        for h in range(H):
            X[:, k * Sp:(k + 1) * Sp, h, :] = 1000 * k + h
    seq = _global_to_seq(X, P)

    def names(block_values):
        return ["S%dH%d" % divmod(int(v), 1000) for v in block_values]

    # before: rank 0's shard lists each head once, in head order
    r0 = seq[0]
    assert names([r0[0, 0, h, 0] for h in range(H)]) == before
    assert (r0 == r0[:, :1, :, :1]).all()  # one tag per head across tokens and dims

    head = oracle.seq_to_head(seq, P)
    assert head.shape == (P, B, S, H // P, D)
    # after: rank 0 holds one block per sequence shard, in sequence order
    blocks = [head[0, 0, k * Sp, 0, 0] for k in range(P)]
    assert names(blocks) == after
    for j in range(P):  # the same statement for every rank j: S0Hj .. S(P-1)Hj
        for k in range(P):
            assert (head[j, :, k * Sp:(k + 1) * Sp] == 1000 * k + j).all()


@pytest.mark.parametrize("B,S,H,D,P", [
    (1, 256, 4, 32, 4), (1, 64, 8, 16, 4), (2, 24, 6, 8, 3), (3, 8, 4, 4, 2),
    (1, 16, 4, 8, 1), (2, 12, 2, 2, 2), (1, 32, 32, 4, 32)])
def test_layout_meaning_by_slicing(B, S, H, D, P):
    """SEQ rank i = tokens of shard i (all heads); HEAD rank j = heads of group j (all tokens)."""
    X = np.arange(B * S * H * D, dtype=np.int64).reshape(B, S, H, D)
    seq = _global_to_seq(X, P)
    want = _global_to_head(X, P)
    got = oracle.seq_to_head(seq, P)
    assert got.shape == (P, B, S, H // P, D)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(oracle.head_to_seq(want, P), seq)


@settings(max_examples=60, deadline=None)
@given(P=st.integers(1, 6), sp=st.integers(0, 5), hp=st.integers(1, 4),
       B=st.integers(0, 3), D=st.integers(1, 9),
       dt=st.sampled_from([np.int8, np.int16, np.int32, np.int64, np.float32]),
       seed=st.integers(0, 2**31))
def test_inverse_identities(P, sp, hp, B, D, dt, seed):
    """head_to_seq . seq_to_head = id and seq_to_head . head_to_seq = id, bitwise."""
    S, H = sp * P, hp * P
    g = np.random.default_rng(seed)
    bits = g.integers(0, 256, size=(P, B, sp, H, D, np.dtype(dt).itemsize), dtype=np.uint8)
    seq = bits.view(dt).reshape(P, B, sp, H, D)
    head = oracle.seq_to_head(seq, P)
    assert head.shape == (P, B, S, hp, D)
    assert oracle.head_to_seq(head, P).tobytes() == seq.tobytes()
    h2 = g.integers(0, 256, size=head.nbytes, dtype=np.uint8).view(dt).reshape(head.shape)
    assert oracle.seq_to_head(oracle.head_to_seq(h2, P), P).tobytes() == h2.tobytes()


def test_bijection_iota():
    """An index tensor comes out as a permutation of itself (every slot written once)."""
    P, B, S, H, D = 8, 2, 64, 16, 8
    n = B * S * H * D
    seq = np.arange(n, dtype=np.int32).reshape(P, B, S // P, H, D)
    head = oracle.seq_to_head(seq, P)
    np.testing.assert_array_equal(np.sort(head.ravel()), np.arange(n, dtype=np.int32))
    # head_dim stays innermost and in order on both sides
    assert (np.diff(head.reshape(-1, D), axis=1) == 1).all()


def test_single_rank_is_identity():
    x = np.random.default_rng(0).standard_normal((1, 2, 10, 3, 5)).astype(np.float32)
    assert oracle.seq_to_head(x, 1).tobytes() == x.tobytes()
    assert oracle.head_to_seq(x, 1).tobytes() == x.tobytes()


def test_nan_payloads_copied_bitwise():
    bits = np.array([0x7FC00001, 0xFFC12345, 0x7F800001, 0x00000001], dtype=np.uint32)
    seq = np.tile(bits, 8).view(np.float32).reshape(2, 1, 2, 2, 4)
    head = oracle.seq_to_head(seq, 2)
    assert sorted(head.view(np.uint32).ravel().tolist()) == sorted(seq.view(np.uint32).ravel().tolist())
    assert oracle.head_to_seq(head, 2).tobytes() == seq.tobytes()


def test_rejects_indivisible():
    with pytest.raises(ValueError):
        oracle.seq_to_head(np.zeros((4, 1, 2, 6, 2), np.float32), 4)  # 6 heads over 4 ranks
    with pytest.raises(ValueError):
        oracle.head_to_seq(np.zeros((4, 1, 6, 1, 2), np.float32), 4)  # 6 tokens over 4 ranks
    with pytest.raises(ValueError):
        oracle.send_bytes(1, 8, 3, 2, 2, 2)


def test_exchange_volumes_match_page(golden_dir):
    """The printed 256/32/28/112/224 MB figures at the pages' shape."""
    g = _parse_kv(os.path.join(golden_dir, "exchange_volumes.txt"))
    P, S, B = int(g["P"]), int(g["S"]), int(g["B"])
    H, D, e = int(g["heads"]), int(g["head_dim"]), int(g["elem_bytes"])
    MB = 1 << 20
    assert B * S * H * D * e == int(g["global_tensor_MB"]) * MB
    assert B * (S // P) * H * D * e == int(g["per_rank_shard_MB"]) * MB
    sends = [oracle.send_bytes(B, S, H, D, P, e, r) for r in (0, 3, P - 1)]
    assert sends == [int(g["send_per_exchange_MB"]) * MB] * 3
    # one exchange each for Q, K, V and the attention output; the same again backward
    assert 4 * sends[0] == int(g["forward_four_exchanges_MB"]) * MB
    assert 8 * sends[0] == int(g["forward_and_backward_MB"]) * MB


def test_send_volume_about_Nd_over_P():
    """Page 1 section 4: a rank sends roughly N*d/P (everything but its own 1/P slice)."""
    for (S, H, D, P) in [(1024, 32, 8, 8), (512, 16, 4, 4), (64, 4, 32, 4), (256, 32, 2, 32)]:
        Nd = S * H * D  # elements of the global activation, one byte each
        sent = oracle.send_bytes(1, S, H, D, P, 1, 0)
        assert sent == Nd // P - Nd // (P * P)
        assert Nd / P * (1 - 1 / P) <= sent <= Nd / P
    assert oracle.send_bytes(1, 64, 4, 8, 1, 2, 0) == 0  # one rank sends nothing


# ---- the exchanges with their pieces left as delivered (no unpack) ----------
# "Sequence Parallelism II..." section 3: every rank cuts its tensor into P
# pieces, piece j goes to rank j, and afterwards each rank holds one piece from
# every rank.  For sequence shards a piece is a head group over the sender's
# tokens; for the attention output it is the receiver's tokens over the
# sender's heads.


def test_worked_rank_map_as_pieces(golden_dir):
    """Page 1's listing again: rank 0's pieces, in order, are S0H0, S1H0, S2H0, S3H0."""
    lines = open(os.path.join(golden_dir, "worked_rank_map.txt")).read()
    P = int(re.search(r"^ranks (\d+)", lines, re.M).group(1))
    H = int(re.search(r"^heads (\d+)", lines, re.M).group(1))
    after = re.search(r"^after 0: (.*)$", lines, re.M).group(1).split()
    S, D, B = 256, 32, 2
    Sp = S // P
    X = np.empty((B, S, H, D), dtype=np.int32)
    for k in range(P):
        for h in range(H):
            X[:, k * Sp:(k + 1) * Sp, h, :] = 1000 * k + h
    pieces = oracle.seq_to_pieces(_global_to_seq(X, P), P)
    assert pieces.shape == (P, P, B, Sp, H // P, D)
    assert ["S%dH%d" % divmod(int(pieces[0, i, 0, 0, 0, 0]), 1000) for i in range(P)] == after
    for j in range(P):
        for i in range(P):
            assert (pieces[j, i] == 1000 * i + j).all()


@pytest.mark.parametrize("B,S,H,D,P", [
    (2, 24, 6, 8, 3), (3, 8, 4, 4, 2), (1, 64, 8, 16, 4), (2, 16, 4, 8, 1), (4, 32, 8, 2, 8)])
def test_pieces_by_slicing(B, S, H, D, P):
    """Piece i of rank j = rank i's tokens over head group j (first exchange); for
    the output, piece i of rank j = rank i's tokens over rank j's heads, and the
    second exchange gives rank i its tokens over every head."""
    Sp, hp = S // P, H // P
    X = np.arange(B * S * H * D, dtype=np.int64).reshape(B, S, H, D)
    got = oracle.seq_to_pieces(_global_to_seq(X, P), P)
    want = np.empty((P, P, B, Sp, hp, D), dtype=X.dtype)
    for j in range(P):
        for i in range(P):
            want[j, i] = X[:, i * Sp:(i + 1) * Sp, j * hp:(j + 1) * hp, :]
    np.testing.assert_array_equal(got, want)
    Y = X[::-1].copy() * 7 + 3  # an attention output over every token and head
    send = np.empty_like(want)
    for j in range(P):
        for i in range(P):
            send[j, i] = Y[:, i * Sp:(i + 1) * Sp, j * hp:(j + 1) * hp, :]
    np.testing.assert_array_equal(oracle.pieces_to_seq(send, P), _global_to_seq(Y, P))


def test_pieces_unpacked_are_the_head_layout():
    """Stacking each rank's pieces along the sequence (per batch entry) is the
    unpacked head layout; for B = 1 the two are the same bytes."""
    g = np.random.default_rng(5)
    for (P, B, Sp, H, D) in [(4, 3, 5, 8, 6), (2, 2, 7, 2, 3), (8, 1, 4, 8, 2)]:
        seq = g.integers(-2**31, 2**31, size=(P, B, Sp, H, D), dtype=np.int32)
        pieces = oracle.seq_to_pieces(seq, P)
        head = oracle.seq_to_head(seq, P)
        unpacked = np.concatenate([pieces[:, i] for i in range(P)], axis=2)
        np.testing.assert_array_equal(unpacked, head)
        if B == 1:
            assert pieces.tobytes() == head.tobytes()


@settings(max_examples=60, deadline=None)
@given(P=st.integers(1, 6), sp=st.integers(0, 5), hp=st.integers(1, 4),
       B=st.integers(0, 3), D=st.integers(1, 9),
       dt=st.sampled_from([np.int8, np.int16, np.int32, np.float32]),
       seed=st.integers(0, 2**31))
def test_pieces_round_trip(P, sp, hp, B, D, dt, seed):
    """pieces_to_seq . seq_to_pieces = id, bitwise (the output's exchange undoes
    the input's when the pieces come back unchanged)."""
    H = hp * P
    g = np.random.default_rng(seed)
    bits = g.integers(0, 256, size=(P, B, sp, H, D, np.dtype(dt).itemsize), dtype=np.uint8)
    seq = bits.view(dt).reshape(P, B, sp, H, D)
    pieces = oracle.seq_to_pieces(seq, P)
    assert pieces.shape == (P, P, B, sp, hp, D)
    assert oracle.pieces_to_seq(pieces, P).tobytes() == seq.tobytes()


def test_pieces_reject_indivisible():
    with pytest.raises(ValueError):
        oracle.seq_to_pieces(np.zeros((4, 1, 2, 6, 2), np.float32), 4)
