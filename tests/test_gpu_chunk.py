"""GPU parity of the key/value-chunk attention and the merge of partial results.

Both are compared with the fp64 oracle (oracle.attention_chunk,
oracle.softmax_merge) on the same seeded inputs:

- chunk outputs within the bf16 bar (max-abs 1e-2, mean-abs 1e-3; fp32 1e-5 /
  1e-6) and lse within 2.5e-3 (bf16: the normaliser is a sum of bf16 weights,
  relative rounding ~2^-9) or 1e-5 (fp32); rows with no visible key must be
  exactly o = 0 and lse = -inf;
- the merge within half a bf16 spacing of the exact result plus fp32 rounding
  of its two terms, lse within 2e-6 relative, empty rows exact;
- a ring over key/value blocks (chunk visits merged in place) against the
  oracle's full attention, at small sizes in full and at the 32k rank shape
  on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (assert_bf16_close, assert_f32_close, dev_bf16, half_ulp_bf16, host_f64,
                     sample_rows)
from sequence_long_context_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sequence_long_context_amd import ulysses as U

LSE_BF16, LSE_F32 = 2.5e-3, 1e-5


def _inputs(seed, B, Sq, Skv, Hq, Hkv, D, dtype):
    q = synth.normal(seed, (B, Sq, Hq, D), dtype)
    k = synth.normal(seed + 1, (B, Skv, Hkv, D), dtype)
    v = synth.normal(seed + 2, (B, Skv, Hkv, D), dtype)
    return q, k, v


def _dev(a, dtype):
    return dev_bf16(a) if dtype == "bf16" else torch.from_numpy(a).cuda()


def _chunk_gpu(q, k, v, causal, q_pos0, k_pos0, dtype):
    qt, kt, vt = (_dev(x, dtype) for x in (q, k, v))
    o = torch.full_like(qt, float("nan"))  # every element must be written
    B, Sq, Hq, _ = qt.shape
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda", dtype=torch.float32)
    U.ulysses_attention_chunk(qt, kt, vt, o, lse, causal, q_pos0, k_pos0)
    return host_f64(o), lse.cpu().numpy().astype(np.float64)


def _check_chunk(got_o, got_l, want_o, want_l, dtype, tag, edge):
    empty = np.isneginf(want_l)  # [B][Hq][Sq]
    assert np.array_equal(np.isneginf(got_l), empty), f"{tag}: empty rows differ"
    e_rows = np.transpose(empty, (0, 2, 1))  # [B][Sq][Hq]
    assert np.all(got_o[e_rows] == 0.0), f"{tag}: empty rows must be 0"
    full = ~e_rows
    if full.any():
        if dtype == "bf16":
            assert_bf16_close(got_o[full], want_o[full], tag, edge=edge)
        else:
            assert_f32_close(got_o[full], want_o[full], tag)
        d = np.abs(got_l[~empty] - want_l[~empty]).max()
        print(f"{tag}: lse max-abs {d:.2e}", flush=True)
        assert d <= (LSE_BF16 if dtype == "bf16" else LSE_F32), tag


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,qp,kp,causal", [
    (1, 256, 256, 2, 2, 0, 0, True),        # the diagonal block: local attention
    (1, 300, 200, 4, 1, 500, 0, True),      # a block entirely in the past: every key
    (2, 333, 257, 2, 2, 100, 150, True),    # rows 0..49 see nothing, then a shifted triangle
    (1, 129, 70, 1, 1, 0, 200, True),       # a block entirely in the future: all rows empty
    (1, 513, 0, 2, 1, 0, 0, True),          # an empty chunk
    (1, 200, 333, 2, 2, 0, 0, False),       # non-causal, different lengths
    (1, 1000, 1000, 4, 2, 1000, 0, True),   # past block, several query blocks
    (1, 64, 1000, 1, 1, 900, 0, True),      # short queries against a long chunk
    (1, 1, 1, 1, 1, 5, 5, True),            # one row, one key
])
def test_bf16_chunk(B, Sq, Skv, Hq, Hkv, qp, kp, causal):
    tag = f"bf16 chunk B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv} q_pos0={qp} k_pos0={kp} causal={causal}"
    print(tag, flush=True)
    q, k, v = _inputs(7 * Sq + 3 * Skv + qp, B, Sq, Skv, Hq, Hkv, 128, "bf16")
    got_o, got_l = _chunk_gpu(q, k, v, causal, qp, kp, "bf16")
    want_o, want_l = oracle.attention_chunk(q, k, v, causal, qp, kp, bf16=True)
    _check_chunk(got_o, got_l, want_o, want_l, "bf16", tag, edge=Skv < 256)


def test_bf16_chunk_paired_blocks():
    """8-wavefront workgroups with paired query blocks (the launch shape of long
    sequences), a ragged chunk and the first 2048 rows without a visible key:
    the short block of a pair is skipped while the long one runs."""
    B, Sq, Skv, Hq, Hkv, qp, kp = 1, 8192, 4000, 16, 4, 2048, 4096
    print(f"bf16 chunk paired Sq={Sq} Skv={Skv} Hq={Hq}", flush=True)
    q, k, v = _inputs(4242, B, Sq, Skv, Hq, Hkv, 128, "bf16")
    got_o, got_l = _chunk_gpu(q, k, v, True, qp, kp, "bf16")
    want_o, want_l = oracle.attention_chunk(q, k, v, True, qp, kp, bf16=True)
    _check_chunk(got_o, got_l, want_o, want_l, "bf16", "paired", edge=False)


def test_bf16_chunk_paired_key_split_ragged():
    """Paired 128-row blocks with the key split (8 heads over 8192 query rows), a key
    count one past a whole tile (8129) and the diagonal shifted so that the short
    blocks see the ragged last tile: the second block of each pair runs right after
    the first block's halves were combined through the tile stages, so the rows past
    the end of that tile must not pick up what the combine left there.  Every row."""
    B, Sq, Skv, Hq, Hkv, qp, kp = 1, 8192, 8129, 8, 2, 8060, 0
    print(f"bf16 chunk paired key split Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv}", flush=True)
    q, k, v = _inputs(5151, B, Sq, Skv, Hq, Hkv, 128, "bf16")
    got_o, got_l = _chunk_gpu(q, k, v, True, qp, kp, "bf16")
    want_o, want_l = oracle.attention_chunk(q, k, v, True, qp, kp, bf16=True)
    _check_chunk(got_o, got_l, want_o, want_l, "bf16", "paired key split ragged", edge=False)


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,qp,kp,causal", [
    (1, 100, 70, 2, 1, 30, 0, True), (1, 77, 130, 1, 1, 0, 50, True),
    (2, 64, 33, 2, 2, 0, 0, False), (1, 40, 20, 1, 1, 0, 100, True), (1, 50, 0, 1, 1, 0, 0, False)])
def test_f32_chunk(D, B, Sq, Skv, Hq, Hkv, qp, kp, causal):
    tag = f"f32 chunk D={D} Sq={Sq} Skv={Skv} q_pos0={qp} k_pos0={kp} causal={causal}"
    print(tag, flush=True)
    q, k, v = _inputs(D + Sq + Skv, B, Sq, Skv, Hq, Hkv, D, "f32")
    got_o, got_l = _chunk_gpu(q, k, v, causal, qp, kp, "f32")
    want_o, want_l = oracle.attention_chunk(q, k, v, causal, qp, kp)
    _check_chunk(got_o, got_l, want_o, want_l, "f32", tag, edge=False)


def _partials(seed, B, S, H, D, dtype):
    """Seeded partial results: o ~ N(0,1); lse ~ N(0, 3^2) with rows empty on one
    side, on the other, and on both (o = 0 there, as the chunk call writes)."""
    oa = synth.normal(seed, (B, S, H, D), dtype)
    ob = synth.normal(seed + 1, (B, S, H, D), dtype)
    la = 3.0 * synth.normal(seed + 2, (B, H, S), "f32")
    lb = 3.0 * synth.normal(seed + 3, (B, H, S), "f32")
    la[:, :, 0::7] = -np.inf
    lb[:, :, 3::7] = -np.inf
    lb[:, :, 0::14] = -np.inf  # both sides empty
    zero = np.uint16(0) if dtype == "bf16" else np.float32(0)
    oa[np.transpose(np.isneginf(la), (0, 2, 1))] = zero
    ob[np.transpose(np.isneginf(lb), (0, 2, 1))] = zero
    return oa, la.astype(np.float32), ob, lb.astype(np.float32)


def _decode(a, dtype):
    return (synth.bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 32), ("f32", 128)])
@pytest.mark.parametrize("inplace", ["none", "a", "b"])
def test_merge(dtype, D, inplace):
    B, S, H = 2, 301, 4
    print(f"merge {dtype} D={D} in place: {inplace}", flush=True)
    oa, la, ob, lb = _partials(90 + D, B, S, H, D, dtype)
    want_o, want_l = oracle.softmax_merge(_decode(oa, dtype), la, _decode(ob, dtype), lb)
    ta, tb = _dev(oa, dtype), _dev(ob, dtype)
    tla, tlb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    if inplace == "a":
        o, lse = ta, tla
    elif inplace == "b":
        o, lse = tb, tlb
    else:
        o, lse = torch.full_like(ta, float("nan")), torch.full_like(tla, float("nan"))
    U.ulysses_attention_merge(ta, tla, tb, tlb, o, lse)
    got_o, got_l = host_f64(o), lse.cpu().numpy().astype(np.float64)

    empty = np.isneginf(want_l)
    assert np.array_equal(np.isneginf(got_l), empty)
    assert np.all(np.abs(got_l[~empty] - want_l[~empty]) <= 2e-6 * np.maximum(1, np.abs(want_l[~empty])))
    # each element: rounding of the output plus fp32 rounding of its two terms
    wa = np.transpose(np.exp(np.where(empty, -np.inf, la - np.where(empty, 0, want_l))), (0, 2, 1))[..., None]
    wb = np.transpose(np.exp(np.where(empty, -np.inf, lb - np.where(empty, 0, want_l))), (0, 2, 1))[..., None]
    terms = wa * np.abs(_decode(oa, dtype)) + wb * np.abs(_decode(ob, dtype))
    bar = (half_ulp_bf16(want_o) if dtype == "bf16" else 0.0) + 1e-6 * terms + 1e-30
    worst = float(np.max(np.abs(got_o - want_o) / bar))
    print(f"merge {dtype}: worst element at {worst:.2f} of its bar", flush=True)
    assert worst <= 1.0
    assert np.all(got_o[np.transpose(empty, (0, 2, 1))] == 0.0)


def _ring_gpu(q, k, v, edges, causal):
    """Each ring rank r keeps query block r and visits the key/value blocks
    r, r-1, ..., r+1 (mod R), merging every visit into its running result in
    place.  Returns o [B][S][Hq][D] and lse [B][Hq][S] of all ranks."""
    qt, kt, vt = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    B, S, Hq, D = qt.shape
    R = len(edges) - 1
    o_all = torch.empty_like(qt)
    lse_all = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
    for r in range(R):
        a, b = edges[r], edges[r + 1]
        qb = qt[:, a:b].contiguous()
        acc_o, acc_l = torch.empty_like(qb), torch.empty((B, Hq, b - a), device="cuda", dtype=torch.float32)
        part_o, part_l = torch.empty_like(acc_o), torch.empty_like(acc_l)
        for t in range(R):
            j = (r - t) % R
            c, d = edges[j], edges[j + 1]
            kb, vb = kt[:, c:d].contiguous(), vt[:, c:d].contiguous()
            dst_o, dst_l = (acc_o, acc_l) if t == 0 else (part_o, part_l)
            U.ulysses_attention_chunk(qb, kb, vb, dst_o, dst_l, causal, a, c)
            if t:
                U.ulysses_attention_merge(acc_o, acc_l, part_o, part_l, acc_o, acc_l)
        o_all[:, a:b] = acc_o
        lse_all[:, :, a:b] = acc_l
    return host_f64(o_all), lse_all.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("edges", [(0, 512, 1024, 1536, 2048), (0, 700, 1300, 2048), (0, 2048)])
def test_ring_equals_attention(edges, causal):
    B, S, Hq, Hkv = 1, 2048, 4, 2
    print(f"ring edges={edges} causal={causal}", flush=True)
    q, k, v = _inputs(5151, B, S, S, Hq, Hkv, 128, "bf16")
    got_o, got_l = _ring_gpu(q, k, v, list(edges), causal)
    want_o, want_l = oracle.attention_chunk(q, k, v, causal, bf16=True)
    assert_bf16_close(got_o, want_o, f"ring {edges}")
    assert np.abs(got_l - want_l).max() <= LSE_BF16


def test_ring_rank_shape_32k_sampled():
    """Ring degree 2 over one Ulysses rank's sequence at the 32k shape (4 heads,
    D = 128, causal): the second ring rank's query half visits its own half
    (the causal diagonal) and the first half (every key), merged in place.
    Compared on sampled rows with the oracle's attention over all keys."""
    B, S, Hq, Hkv = 1, 32768, 4, 4
    h = S // 2
    print("ring s32k rank 1 of 2", flush=True)
    q, k, v = _inputs(3001, B, S, S, Hq, Hkv, 128, "bf16")
    qt, kt, vt = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    qb = qt[:, h:].contiguous()
    o, lse = torch.empty_like(qb), torch.empty((B, Hq, h), device="cuda", dtype=torch.float32)
    po, pl = torch.empty_like(o), torch.empty_like(lse)
    U.ulysses_attention_chunk(qb, kt[:, h:].contiguous(), vt[:, h:].contiguous(), o, lse, True, h, h)
    U.ulysses_attention_chunk(qb, kt[:, :h].contiguous(), vt[:, :h].contiguous(), po, pl, True, h, 0)
    U.ulysses_attention_merge(o, lse, po, pl, o, lse)
    got_o, got_l = host_f64(o), lse.cpu().numpy().astype(np.float64)
    rows = sample_rows(h, 8, 24, seed=11)
    want_o = np.empty((B, len(rows), Hq, 128))
    want_l = np.empty((B, Hq, len(rows)))
    for n, i in enumerate(rows):
        wo, wl = oracle.attention_chunk(q[:, h + i:h + i + 1], k, v, True, q_pos0=h + i, bf16=True)
        want_o[:, n], want_l[:, :, n] = wo[:, 0], wl[:, :, 0]
    assert_bf16_close(got_o[:, rows], want_o, "ring s32k sampled rows")
    assert np.abs(got_l[:, :, rows] - want_l).max() <= LSE_BF16


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,qp,kp,causal", [
    (1, 300, 256, 2, 2, 300, 300, True),    # the diagonal block (Sq > Skv: rows 256.. see all)
    (1, 300, 200, 4, 1, 500, 0, True),      # a block from the past
    (2, 333, 257, 2, 2, 100, 150, True),    # first 50 rows see nothing: unchanged
    (1, 129, 70, 1, 1, 0, 200, True),       # a block from the future: nothing changes
    (1, 200, 0, 2, 1, 0, 0, False),         # an empty chunk: nothing changes
    (1, 2000, 1500, 4, 2, 1500, 0, False),  # non-causal, several blocks
    (1, 8192, 4000, 16, 4, 2048, 4096, True),  # 256-row pairs, first 2048 rows unchanged
])
def test_chunk_accumulate(B, Sq, Skv, Hq, Hkv, qp, kp, causal):
    """(o, lse) = merge(running result, this chunk) in one launch, against the oracle's
    chunk attention merged by the oracle; rows the chunk does not reach keep their bits."""
    tag = f"accumulate B={B} Sq={Sq} Skv={Skv} q_pos0={qp} k_pos0={kp} causal={causal}"
    print(tag, flush=True)
    q, k, v = _inputs(31 * Sq + Skv, B, Sq, Skv, Hq, Hkv, 128, "bf16")
    oa, la, _, _ = _partials(17 + Sq, B, Sq, Hq, 128, "bf16")
    la = np.where(np.isneginf(la), la, la + 3.0).astype(np.float32)  # comparable to the chunk's lse
    want_c, want_cl = oracle.attention_chunk(q, k, v, causal, qp, kp, bf16=True)
    want_o, want_l = oracle.softmax_merge(_decode(oa, "bf16"), la, want_c, want_cl)
    o, lse = dev_bf16(oa), torch.from_numpy(la).cuda()
    U.ulysses_attention_chunk_accumulate(dev_bf16(q), dev_bf16(k), dev_bf16(v), o, lse, causal, qp, kp)
    got_o, got_l = host_f64(o), lse.cpu().numpy().astype(np.float64)
    untouched = np.isneginf(want_cl)  # [B][Hq][Sq]: this chunk reaches no key of the row
    assert np.array_equal(got_l[untouched], la[untouched].astype(np.float64)), tag
    rows = np.transpose(untouched, (0, 2, 1))
    assert np.array_equal(got_o[rows], _decode(oa, "bf16")[rows]), tag
    if (~rows).any():
        # the running result is N(0,1) (magnitudes up to ~4), so the merged bf16
        # output carries up to half a bf16 spacing of rounding on top of the
        # chunk's error: the edge-case bar (1e-2 plus half a spacing)
        assert_bf16_close(got_o[~rows], want_o[~rows], tag, edge=True)
        assert np.abs(got_l[~untouched] - want_l[~untouched]).max() <= LSE_BF16, tag


@pytest.mark.parametrize("causal", [True, False])
def test_ring_accumulate_equals_attention(causal):
    """A ring of four visits: the first with ulysses_attention_chunk, the other three
    merged in the same launch; equal to the oracle's attention over all keys."""
    B, S, Hq, Hkv = 1, 2048, 4, 2
    edges = [0, 500, 1024, 1600, 2048]
    print(f"ring accumulate causal={causal}", flush=True)
    q, k, v = _inputs(6161, B, S, S, Hq, Hkv, 128, "bf16")
    qt, kt, vt = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o_all = torch.empty_like(qt)
    lse_all = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
    R = len(edges) - 1
    for r in range(R):
        a, b = edges[r], edges[r + 1]
        qb = qt[:, a:b].contiguous()
        o = torch.empty_like(qb)
        lse = torch.empty((B, Hq, b - a), device="cuda", dtype=torch.float32)
        for t in range(R):
            j = (r - t) % R
            c, d = edges[j], edges[j + 1]
            fn = U.ulysses_attention_chunk if t == 0 else U.ulysses_attention_chunk_accumulate
            fn(qb, kt[:, c:d].contiguous(), vt[:, c:d].contiguous(), o, lse, causal, a, c)
        o_all[:, a:b] = o
        lse_all[:, :, a:b] = lse
    want_o, want_l = oracle.attention_chunk(q, k, v, causal, bf16=True)
    assert_bf16_close(host_f64(o_all), want_o, f"ring accumulate causal={causal}")
    assert np.abs(lse_all.cpu().numpy() - want_l).max() <= LSE_BF16


@pytest.mark.parametrize("causal", [True, False])
def test_ulysses_ring_hybrid_past_head_count(causal):
    """Sequence parallelism over 16 ranks with 8 heads (twice the head-count bound):
    two ring groups of 8 Ulysses ranks.  Group g owns sequence half g; inside it
    the seq->head exchange gives rank j head j over that half; the two groups'
    key/value halves then circulate (a ring of degree 2 per head: each query half
    visits its own half and the other, merged in the same launch); head->seq
    returns the output.  Equal to multi-head attention over the whole sequence."""
    B, S, H, D, P, R = 1, 2048, 8, 128, 8, 2
    Sh = S // R
    print(f"Ulysses x ring hybrid P={P} R={R} heads={H} causal={causal}", flush=True)
    x = {t: synth.normal(900 + i, (B, S, H, D)) for i, t in enumerate("qkv")}
    head = {}
    for t in "qkv":  # per ring group: [P][B][Sh][1][D] (rank j = head j over half g)
        head[t] = []
        for g in range(R):
            seq = dev_bf16(np.ascontiguousarray(x[t][:, g * Sh:(g + 1) * Sh]).reshape(P, B, Sh // P, H, D))
            dst = torch.empty((P, B, Sh, H // P, D), dtype=torch.bfloat16, device="cuda")
            head[t].append(U.ulysses_seq_to_head(seq, dst, P))
    out = np.empty((B, S, H, D))
    for g in range(R):
        o_head = torch.empty((P, B, Sh, H // P, D), dtype=torch.bfloat16, device="cuda")
        for j in range(P):
            o = o_head[j]
            lse = torch.empty((B, H // P, Sh), dtype=torch.float32, device="cuda")
            for t in range(R):
                gk = (g - t) % R
                fn = U.ulysses_attention_chunk if t == 0 else U.ulysses_attention_chunk_accumulate
                fn(head["q"][g][j], head["k"][gk][j], head["v"][gk][j], o, lse, causal, g * Sh, gk * Sh)
        o_seq = torch.empty((P, B, Sh // P, H, D), dtype=torch.bfloat16, device="cuda")
        U.ulysses_head_to_seq(o_head, o_seq, P)
        out[:, g * Sh:(g + 1) * Sh] = host_f64(o_seq).reshape(B, Sh, H, D)
    want = oracle.attention(x["q"], x["k"], x["v"], causal, bf16=True)
    assert_bf16_close(out, want, f"hybrid causal={causal}")
