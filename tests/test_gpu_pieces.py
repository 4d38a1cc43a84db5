"""GPU parity of the exchanges with their pieces left as delivered, and of the
attention that reads and writes that order, against the oracle.

Layout calls are bit-exact against oracle.seq_to_pieces / pieces_to_seq.  The
attention on one rank's pieces [P][B][S/P][h][D] is compared with the oracle's
attention of the same rank's heads in [B][S][h][D] order (unpacked here by a
numpy transpose), to the forward bars (bf16: max-abs 1e-2, mean-abs 1e-3;
fp32: 1e-5 / 1e-6), and bit for bit with ulysses_attention_local on the
unpacked buffers (the same kernel arithmetic; only addresses differ).  Batch
sizes 2 and 3 are where the two orders differ; pieces of 192 rows put a
query block across a piece boundary.  The gradient call in piece order is
checked the same way: bit for bit against the plain gradient call on the
unpacked buffers, and against the oracle's gradients to the gradient bars.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (assert_bf16_close, assert_f32_close, dev_bf16, dev_raw, host_bits, host_f64,
                     stratified_rows)
from sequence_long_context_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sequence_long_context_amd import ulysses as U


def unpack(x):
    """One rank's pieces [P][B][S/P][h][D] -> [B][S][h][D] (piece i = tokens of rank i)."""
    P, B, Sp, h, D = x.shape
    return np.ascontiguousarray(np.transpose(x, (1, 0, 2, 3, 4)).reshape(B, P * Sp, h, D))


def pack(x, P):
    """[B][S][h][D] -> [P][B][S/P][h][D]."""
    B, S, h, D = x.shape
    return np.ascontiguousarray(np.transpose(x.reshape(B, P, S // P, h, D), (1, 0, 2, 3, 4)))


# ---- layout ----------------------------------------------------------------------

@pytest.mark.parametrize("P,B,S,H,D,et", [
    (4, 3, 64, 8, 128, np.int16), (8, 2, 1024, 32, 128, np.int16), (2, 2, 10, 6, 3, np.int32),
    (1, 2, 8, 4, 16, np.int16), (3, 3, 9, 3, 5, np.int16), (8, 1, 512, 8, 128, np.int16),
    (4, 2, 4096, 4, 128, np.int32)])
def test_layout_bit_exact(P, B, S, H, D, et):
    print(f"pieces layout P={P} B={B} S={S} H={H} D={D} {np.dtype(et).name}", flush=True)
    g = np.random.default_rng(S * 31 + H * 7 + B)
    seq = g.integers(np.iinfo(et).min, np.iinfo(et).max, size=(P, B, S // P, H, D), dtype=et,
                     endpoint=True)
    src = dev_raw(seq)
    dst = torch.empty((P, P, B, S // P, H // P, D), dtype=src.dtype, device="cuda")
    U.ulysses_seq_to_pieces(src, dst, P)
    assert host_bits(dst).tobytes() == oracle.seq_to_pieces(seq, P).tobytes()
    pieces = g.integers(np.iinfo(et).min, np.iinfo(et).max, size=(P, P, B, S // P, H // P, D),
                        dtype=et, endpoint=True)
    back = torch.empty((P, B, S // P, H, D), dtype=src.dtype, device="cuda")
    U.ulysses_pieces_to_seq(dev_raw(pieces), back, P)
    assert host_bits(back).tobytes() == oracle.pieces_to_seq(pieces, P).tobytes()


@pytest.mark.parametrize("P,B,S,Hq,Hkv,D", [(4, 3, 256, 8, 4, 128), (8, 2, 512, 32, 8, 128),
                                            (2, 2, 6, 4, 2, 3)])
def test_layout_qkv_bit_exact(P, B, S, Hq, Hkv, D):
    print(f"pieces layout qkv P={P} B={B} S={S} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
    g = np.random.default_rng(S + Hq)
    seqs = [g.integers(-2**15, 2**15, size=(P, B, S // P, H, D), dtype=np.int16)
            for H in (Hq, Hkv, Hkv)]
    src = [dev_raw(x) for x in seqs]
    dst = [torch.full((P, P, B, S // P, H // P, D), -1, dtype=torch.int16, device="cuda")
           for H in (Hq, Hkv, Hkv)]
    U.ulysses_seq_to_pieces_qkv(*src, *dst, P)
    for x, d in zip(seqs, dst):
        assert host_bits(d).tobytes() == oracle.seq_to_pieces(x, P).tobytes()


def test_layout_empty_is_noop():
    src = torch.zeros((4, 0, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    dst = torch.zeros((4, 4, 0, 16, 2, 128), dtype=torch.bfloat16, device="cuda")
    U.ulysses_seq_to_pieces(src, dst, 4)
    U.ulysses_pieces_to_seq(dst, src, 4)


# ---- attention on pieces -------------------------------------------------------------

def _pieces_attention_gpu(qp, kp, vp, causal, dt):
    up = dev_bf16 if dt == "bf16" else (lambda a: torch.from_numpy(a).cuda())
    q, k, v = up(qp), up(kp), up(vp)
    P, B, Sp, Hq, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, P * Sp), dtype=torch.float32, device="cuda")
    U.ulysses_attention_local_pieces(q, k, v, o, causal, lse)
    o2 = torch.empty_like(q)  # without lse
    U.ulysses_attention_local_pieces(q, k, v, o2, causal)
    # the plain call on the unpacked buffers
    qu, ku, vu = (x.permute(1, 0, 2, 3, 4).reshape(B, P * Sp, -1, D).contiguous() for x in (q, k, v))
    ou = torch.empty_like(qu)
    lu = torch.empty_like(lse)
    U.ulysses_attention_local_lse(qu, ku, vu, ou, lu, causal)
    ou_packed = ou.view(B, P, Sp, Hq, D).permute(1, 0, 2, 3, 4).contiguous()
    assert host_bits(o).tobytes() == host_bits(ou_packed).tobytes(), "differs from the plain call"
    assert host_bits(o2).tobytes() == host_bits(o).tobytes(), "lse changes the output"
    assert host_bits(lse).tobytes() == host_bits(lu).tobytes(), "lse differs from the plain call"
    return host_f64(o)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,S,P,Hq,Hkv", [
    (2, 1024, 8, 8, 2), (3, 768, 4, 4, 4), (2, 4096, 8, 4, 1), (3, 384, 6, 2, 2), (2, 128, 2, 1, 1)])
def test_bf16_pieces(B, S, P, Hq, Hkv, causal):
    print(f"bf16 attention on pieces B={B} S={S} P={P} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    seed = 7 * S + 3 * B + Hq
    qp = synth.normal(seed, (P, B, S // P, Hq, 128))
    kp = synth.normal(seed + 1, (P, B, S // P, Hkv, 128))
    vp = synth.normal(seed + 2, (P, B, S // P, Hkv, 128))
    got = _pieces_attention_gpu(qp, kp, vp, causal, "bf16")
    want = oracle.attention(unpack(qp), unpack(kp), unpack(vp), causal, bf16=True)
    assert_bf16_close(unpack(got), want, f"pieces B={B} S={S} P={P} causal={causal}")


@pytest.mark.parametrize("causal", [True, False])
def test_bf16_one_batch_entry_any_piece_height(causal):
    """B = 1: the pieces are the sequence order, so pieces of any height (125 rows) work."""
    B, S, P, H = 1, 1000, 8, 2
    qp, kp, vp = (synth.normal(900 + i, (P, B, S // P, H, 128)) for i in range(3))
    got = _pieces_attention_gpu(qp, kp, vp, causal, "bf16")
    want = oracle.attention(unpack(qp), unpack(kp), unpack(vp), causal, bf16=True)
    assert_bf16_close(unpack(got), want, f"pieces B=1 S={S} P={P} causal={causal}")


@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,S,P,Hq,Hkv", [(3, 96, 8, 4, 2), (2, 60, 4, 2, 2), (2, 200, 5, 1, 1)])
def test_fp32_pieces(B, S, P, Hq, Hkv, causal, D):
    print(f"fp32 attention on pieces B={B} S={S} P={P} D={D} causal={causal}", flush=True)
    seed = 11 * S + D + B
    qp, kp, vp = (synth.normal(seed + i, (P, B, S // P, h, D), "f32")
                  for i, h in enumerate((Hq, Hkv, Hkv)))
    got = _pieces_attention_gpu(qp, kp, vp, causal, "f32")
    want = oracle.attention(unpack(qp), unpack(kp), unpack(vp), causal)
    assert_f32_close(unpack(got), want, f"fp32 pieces B={B} S={S} P={P} D={D} causal={causal}")


def test_bf16_pieces_shorter_than_a_tile_rejected():
    q = torch.zeros((3, 2, 32, 2, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(U.UlyssesError, match="multiple of 64") as err:
        U.ulysses_attention_local_pieces(q, q, q, o, True)
    assert err.value.status == U.ULY_ERR_UNSUPPORTED


# ---- the whole path in pieces order -----------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_whole_path_in_pieces(causal):
    """seq -> pieces (Q, K, V in one launch), attention on every rank's pieces, pieces -> seq:
    against the oracle's exchanges and attention, and bit for bit against the path
    through the head layout."""
    P, B, S, Hq, Hkv = 4, 2, 1024, 16, 4
    hq, hkv = Hq // P, Hkv // P
    print(f"whole path in pieces P={P} B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    seqs = [synth.normal(300 + i, (P, B, S // P, H, 128)) for i, H in enumerate((Hq, Hkv, Hkv))]
    src = [dev_bf16(x) for x in seqs]
    pcs = [torch.empty((P, P, B, S // P, H // P, 128), dtype=torch.bfloat16, device="cuda")
           for H in (Hq, Hkv, Hkv)]
    U.ulysses_seq_to_pieces_qkv(*src, *pcs, P)
    o_p = torch.empty_like(pcs[0])
    for r in range(P):
        U.ulysses_attention_local_pieces(pcs[0][r], pcs[1][r], pcs[2][r], o_p[r], causal)
    o_seq = torch.empty_like(src[0])
    U.ulysses_pieces_to_seq(o_p, o_seq, P)

    heads = [torch.empty((P, B, S, H // P, 128), dtype=torch.bfloat16, device="cuda")
             for H in (Hq, Hkv, Hkv)]
    U.ulysses_seq_to_head_qkv(*src, *heads, P)
    o_h = torch.empty_like(heads[0])
    for r in range(P):
        U.ulysses_attention_local(heads[0][r], heads[1][r], heads[2][r], o_h[r], causal)
    o_seq2 = torch.empty_like(src[0])
    U.ulysses_head_to_seq(o_h, o_seq2, P)
    assert host_bits(o_seq).tobytes() == host_bits(o_seq2).tobytes()

    # oracle: exchange, attention per rank on its unpacked pieces, exchange back
    qo, ko, vo = (oracle.seq_to_pieces(x, P) for x in seqs)
    out_pieces = np.empty((P, P, B, S // P, hq, 128))
    for r in range(P):
        o_r = oracle.attention(unpack(qo[r]), unpack(ko[r]), unpack(vo[r]), causal, bf16=True)
        out_pieces[r] = pack(o_r, P)
    want = oracle.pieces_to_seq(out_pieces, P)
    assert_bf16_close(host_f64(o_seq), want, f"whole path in pieces causal={causal}")


def test_bf16_pieces_long_stratified():
    """One rank's share of the 32k-token workload as two batch entries of 16384
    tokens (4 query heads, 4 kv heads, P = 8): computed in full, compared with the
    oracle on 1024 stratified rows per batch entry and head."""
    B, S, P, H = 2, 16384, 8, 4
    print(f"bf16 attention on pieces B={B} S={S} P={P} H={H} causal", flush=True)
    qp, kp, vp = (synth.normal(4000 + i, (P, B, S // P, H, 128)) for i in range(3))
    q, k, v = dev_bf16(qp), dev_bf16(kp), dev_bf16(vp)
    o = torch.empty_like(q)
    U.ulysses_attention_local_pieces(q, k, v, o, True)
    rows = stratified_rows(S, P, 1024, 17)
    assert rows.size >= 1024
    got = unpack(host_f64(o))[:, rows]
    want = oracle.attention(unpack(qp), unpack(kp), unpack(vp), True, bf16=True, rows=rows)
    assert_bf16_close(got, want, f"pieces long B={B} S={S}")


# ---- gradients in piece order -----------------------------------------------------------

def _assert_grad_close(got, ref, what):
    """max |GPU - oracle| <= 1 % of the largest |oracle| element, mean <= 0.5 % of the mean
    (the bars of the gradient parity tests)."""
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = err.max(initial=0.0), err.mean() if err.size else 0.0
    big, avg = np.abs(ref).max(initial=0.0), np.abs(ref).mean() if ref.size else 0.0
    print(f"{what}: max {mx:.3e} (bar {1e-2 * big:.3e}) mean {mean:.3e} (bar {5e-3 * avg:.3e})", flush=True)
    assert mx <= 1e-2 * big + 1e-6 and mean <= 5e-3 * avg + 1e-7, what


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,S,P,Hq,Hkv", [(2, 1024, 8, 8, 2), (3, 768, 4, 4, 4), (2, 128, 2, 1, 1)])
def test_backward_pieces(B, S, P, Hq, Hkv, causal):
    print(f"gradients on pieces B={B} S={S} P={P} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    seed = 13 * S + 5 * B + Hq
    qp, kp, vp = (synth.normal(seed + i, (P, B, S // P, h, 128)) for i, h in enumerate((Hq, Hkv, Hkv)))
    gp = synth.normal(seed + 3, (P, B, S // P, Hq, 128))
    q, k, v, g = dev_bf16(qp), dev_bf16(kp), dev_bf16(vp), dev_bf16(gp)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    U.ulysses_attention_local_pieces(q, k, v, o, causal, lse)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    U.ulysses_attention_local_backward_pieces(q, k, v, o, g, lse, delta, dq, dk, dv, causal)
    # the plain call on unpacked buffers
    up = [x.permute(1, 0, 2, 3, 4).reshape(B, S, -1, 128).contiguous() for x in (q, k, v, o, g)]
    lse2, delta2 = torch.empty_like(lse), torch.empty_like(lse)
    U.ulysses_attention_local_lse(up[0], up[1], up[2], torch.empty_like(up[0]), lse2, causal)
    pq, pk, pv = (torch.empty_like(x) for x in up[:3])
    U.ulysses_attention_local_backward(up[0], up[1], up[2], up[3], up[4], lse, delta2, pq, pk, pv, causal)
    for name, a, b in (("dq", dq, pq), ("dk", dk, pk), ("dv", dv, pv)):
        packed = b.view(B, P, S // P, -1, 128).permute(1, 0, 2, 3, 4).contiguous()
        assert host_bits(a).tobytes() == host_bits(packed).tobytes(), f"{name} differs from the plain call"
    assert host_bits(delta).tobytes() == host_bits(delta2).tobytes()
    assert host_bits(lse).tobytes() == host_bits(lse2).tobytes()
    # against the oracle, unpacked (delta from the oracle's output rounded to bf16)
    ref = oracle.attention_backward(unpack(qp), unpack(kp), unpack(vp), unpack(gp), causal, bf16=True,
                                    round_o=True)
    for name, a, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        _assert_grad_close(unpack(host_f64(a)), r, f"{name} pieces B={B} S={S} causal={causal}")


def test_backward_pieces_shorter_than_a_tile_rejected():
    q = torch.zeros((3, 2, 32, 2, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, 2, 96), dtype=torch.float32, device="cuda")
    with pytest.raises(U.UlyssesError, match="multiple of 64") as err:
        U.ulysses_attention_local_backward_pieces(q, q, q, q, q, lse, lse.clone(), q.clone(), q.clone(),
                                                  q.clone(), True)
    assert err.value.status == U.ULY_ERR_UNSUPPORTED
