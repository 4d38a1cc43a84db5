"""GPU parity of the attention gradients (and of the forward's log-sum-exp) against the fp64 oracle.

Tolerances, from the arithmetic.  The gradient call takes delta from the bf16
output o it is given.  Checks are made against the oracle's derivative with
delta taken from its own output rounded to bf16 (round_o, the contract of the
call) and, from 64 keys on, also against the exact derivative (delta from the
exact output), whose distance from the contract is the rounding of delta: at
most 0.43 % of the largest element from S = 64, but up to 1.9 % with two keys,
where only the contract is checked.  Beyond
that the kernels round the softmax weights P and dS to bf16 (relative 2^-9,
round to nearest even) before their products, accumulate in fp32 and round dQ,
dK, dV to bf16 (2^-9).  A handful of 2^-9 (0.2 %) contributions per element
gives the bounds used here: max |GPU - oracle| <= 1 % of the largest |oracle|
element, mean <= 0.5 % of the mean |oracle| element.  The forward's row sum adds
the bf16-rounded weights, so its log-sum-exp is within log(1 + 2^-9) < 2.5e-3 of
the exact one.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import dev_bf16, host_f64
from sequence_long_context_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sequence_long_context_amd import ulysses as U

MAX_REL, MEAN_REL, LSE_ABS = 1e-2, 5e-3, 2.5e-3


def _grads_gpu(qb, kb, vb, gb, causal):
    q, k, v, g = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    B, S, Hq, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device=q.device, dtype=torch.float32)
    U.ulysses_attention_local_lse(q, k, v, o, lse, causal)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    U.ulysses_attention_local_backward(q, k, v, o, g, lse, delta, dq, dk, dv, causal)
    return host_f64(dq), host_f64(dk), host_f64(dv), lse.cpu().numpy().astype(np.float64)


def _assert_grad_close(got, ref, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = err.max(initial=0.0), err.mean() if err.size else 0.0
    big, avg = np.abs(ref).max(initial=0.0), np.abs(ref).mean() if ref.size else 0.0
    assert mx <= MAX_REL * big + 1e-6, f"{what}: max err {mx:.3e} > {MAX_REL} * {big:.3e}"
    assert mean <= MEAN_REL * avg + 1e-7, f"{what}: mean err {mean:.3e} > {MEAN_REL} * {avg:.3e}"


def _derivatives(S):
    """round_o settings to compare against: the call's contract (delta from the bf16
    output it receives) always; the exact derivative from 64 keys on -- with one or
    two keys the rounding of o to bf16 alone moves dQ and dK by up to 1.9 % of their
    largest element (measured with the oracle at S = 2, causal; at most 0.43 % from
    S = 64), so there only the contract can hold."""
    return (True, False) if S >= 64 else (True,)


def _check(qb, kb, vb, gb, causal, tag):
    got = _grads_gpu(qb, kb, vb, gb, causal)
    for round_o in _derivatives(qb.shape[1]):
        ref = oracle.attention_backward(qb, kb, vb, gb, causal, bf16=True, round_o=round_o)
        for name, a, b in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            _assert_grad_close(a, b, f"{tag} {name} (round_o={round_o})")
        assert np.abs(got[3] - ref[3]).max() <= LSE_ABS, f"{tag} lse"


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,S,Hq,Hkv", [
    (1, 1, 1, 1), (1, 2, 1, 1), (1, 64, 2, 2), (1, 65, 1, 1), (1, 130, 2, 1), (2, 200, 4, 2),
    (1, 300, 2, 2), (1, 512, 4, 4), (1, 256, 8, 2), (1, 1000, 4, 1), (3, 129, 2, 2)])
def test_backward_small_full(B, S, Hq, Hkv, causal):
    print(f"bf16 backward B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    seed = 7 * S + 3 * Hq + Hkv + 11 * B
    qb, gb = synth.normal(seed, (B, S, Hq, 128)), synth.normal(seed + 3, (B, S, Hq, 128))
    kb, vb = synth.normal(seed + 1, (B, S, Hkv, 128)), synth.normal(seed + 2, (B, S, Hkv, 128))
    _check(qb, kb, vb, gb, causal, f"B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}")


def test_backward_s4k_full():
    """S = 4096, 4 heads (the short workload's rank shape), both masks, every element."""
    for causal in (True, False):
        print(f"bf16 backward S=4096 H=4 causal={causal}", flush=True)
        qb, gb = synth.normal(901, (1, 4096, 4, 128)), synth.normal(904, (1, 4096, 4, 128))
        kb, vb = synth.normal(902, (1, 4096, 4, 128)), synth.normal(903, (1, 4096, 4, 128))
        _check(qb, kb, vb, gb, causal, f"S=4096 causal={causal}")


def test_backward_many_heads():
    """128 heads over B = 2 (more dK/dV workgroups than CUs), three key blocks with a ragged
    end, causal. Every element."""
    B, S, H = 2, 380, 64
    print(f"bf16 backward many heads B={B} S={S} H={H}", flush=True)
    qb, gb = synth.normal(911, (B, S, H, 128)), synth.normal(914, (B, S, H, 128))
    kb, vb = synth.normal(912, (B, S, H, 128)), synth.normal(913, (B, S, H, 128))
    _check(qb, kb, vb, gb, True, f"many heads B={B} S={S} H={H}")


def test_backward_rows_past_end_ignored():
    """Rows after batch 0's ragged end (batch 1's, filled with NaN/Inf) never reach batch 0's gradients."""
    B, S, H = 2, 100, 2
    qb, gb = synth.normal(61, (B, S, H, 128)), synth.normal(64, (B, S, H, 128))
    kb, vb = synth.normal(62, (B, S, H, 128)), synth.normal(63, (B, S, H, 128))
    for x in (qb, kb, vb, gb):
        x[1] = np.uint16(0x7FC0)  # NaN
    kb[1, :, 0] = np.uint16(0x7F80)  # +Inf
    for causal in (True, False):
        got = _grads_gpu(qb, kb, vb, gb, causal)
        for round_o in (True, False):
            ref = oracle.attention_backward(qb[:1], kb[:1], vb[:1], gb[:1], causal, bf16=True,
                                            round_o=round_o)
            for name, a, b in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
                _assert_grad_close(a[:1], b, f"rows past the end causal={causal} {name} (round_o={round_o})")


def test_backward_deterministic():
    qb, gb = synth.normal(81, (1, 777, 4, 128)), synth.normal(84, (1, 777, 4, 128))
    kb, vb = synth.normal(82, (1, 777, 2, 128)), synth.normal(83, (1, 777, 2, 128))
    a = _grads_gpu(qb, kb, vb, gb, True)
    b = _grads_gpu(qb, kb, vb, gb, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_fp32_lse(D):
    g = np.random.default_rng(D)
    S, Hq, Hkv = 150, 2, 1
    q = g.standard_normal((1, S, Hq, D)).astype(np.float32)
    k = g.standard_normal((1, S, Hkv, D)).astype(np.float32)
    v = g.standard_normal((1, S, Hkv, D)).astype(np.float32)
    for causal in (True, False):
        qt, kt, vt = (torch.from_numpy(x).cuda() for x in (q, k, v))
        o = torch.empty_like(qt)
        lse = torch.empty((1, Hq, S), device="cuda", dtype=torch.float32)
        U.ulysses_attention_local_lse(qt, kt, vt, o, lse, causal)
        ref = oracle.attention_backward(q, k, v, np.zeros_like(q), causal)[3]
        np.testing.assert_allclose(lse.cpu().numpy(), ref, rtol=0, atol=1e-5)
        np.testing.assert_allclose(host_f64(o), oracle.attention(q, k, v, causal), rtol=0, atol=1e-5)


def test_backward_unsupported_fp32():
    t = torch.zeros((1, 8, 1, 32), device="cuda", dtype=torch.float32)
    lse = torch.zeros((1, 1, 8), device="cuda", dtype=torch.float32)
    with pytest.raises(U.UlyssesError) as e:
        U.ulysses_attention_local_backward(t, t.clone(), t.clone(), t.clone(), t.clone(), lse,
                                           lse.clone(), t.clone(), t.clone(), t.clone(), True)
    assert e.value.status == U.ULY_ERR_UNSUPPORTED


@pytest.mark.parametrize("S,Hq,Hkv,seed", [(8192, 4, 4, 950), (6144, 8, 2, 960)])
def test_backward_one_launch_mid(S, Hq, Hkv, seed):
    """Mid lengths whose dQ grid is unpaired: the dQ and dK/dV workgroups share one launch,
    ordered longest first, with more workgroups than compute units (S = 8192 with 4 heads:
    512; S = 6144 with 8 query heads on 2 kv heads: 480).  Causal; dQ on 512 rows spread over
    the sequence, dK and dV on one key in every 128-key block (every dK/dV workgroup),
    against the oracle's sampled gradients."""
    from helpers import stratified_rows
    print(f"one-launch backward S={S} Hq={Hq} Hkv={Hkv}", flush=True)
    qb, gb = synth.normal(seed, (1, S, Hq, 128)), synth.normal(seed + 3, (1, S, Hq, 128))
    kb, vb = synth.normal(seed + 1, (1, S, Hkv, 128)), synth.normal(seed + 2, (1, S, Hkv, 128))
    dq, dk, dv, _ = _grads_gpu(qb, kb, vb, gb, True)
    rows = stratified_rows(S, 8, 512, seed)
    keys = stratified_rows(S, 8, S // 128, seed + 100)
    rq, rk, rv = oracle.attention_backward_sampled(qb, kb, vb, gb, True, rows, keys, bf16=True,
                                                   round_o=True)
    _assert_grad_close(dq[:, rows], rq, f"S={S} dq ({rows.size} rows)")
    _assert_grad_close(dk[:, keys], rk, f"S={S} dk ({keys.size} keys)")
    _assert_grad_close(dv[:, keys], rv, f"S={S} dv ({keys.size} keys)")


@pytest.mark.parametrize("name,S,Hq,Hkv,exact", [
    ("s32k_4heads", 32768, 4, 4, True),
    ("s64k_gqa_4q1kv", 65536, 4, 1, False),
])
def test_backward_long_sampled(name, S, Hq, Hkv, exact):
    """Gradients at the long workloads' rank shapes (causal), in the configuration the bench
    times: dQ on 1024 rows spread over the sequence (plus row 0, 1, S-1 and every rank
    boundary); dK and dV on one key in every 128-key block (the dK/dV kernel's blocks),
    key 0, S-1 and every rank boundary -- early keys are seen by the long query streams
    that dominate that kernel (at 64k: the blocks of the last eighth); and all of dK and
    dV through two exact identities: the
    value gradients of a kv head add up to the summed output gradients of its query heads
    (the weights of a row sum to one), and the key gradients add up to zero (the dS of a
    row sum to zero).  At 32k also against the exact derivative."""
    print(f"long backward {name}", flush=True)
    from helpers import stratified_rows
    wl = {"s32k_4heads": 2, "s64k_gqa_4q1kv": 3}[name]
    qb = synth.normal(synth.seed_for(wl, "q"), (1, S, Hq, 128))
    kb = synth.normal(synth.seed_for(wl, "k"), (1, S, Hkv, 128))
    vb = synth.normal(synth.seed_for(wl, "v"), (1, S, Hkv, 128))
    gb = synth.normal(synth.seed_for(wl, "do"), (1, S, Hq, 128))
    dq, dk, dv, _ = _grads_gpu(qb, kb, vb, gb, True)
    for name_, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.isfinite(x).all(), name_
    rows = stratified_rows(S, 8, 1024, wl)
    if exact:  # one key in every 128-key block of the sequence
        keys = stratified_rows(S, 8, S // 128, wl + 100)
    else:  # grouped heads on one kv head: the same over the last eighth (the oracle's
        # cost grows with the rows that see the earliest listed key)
        keys = 7 * S // 8 + stratified_rows(S // 8, 1, S // 8 // 128, wl + 100)
    for round_o in ((True, False) if exact else (True,)):
        rq, rk, rv = oracle.attention_backward_sampled(qb, kb, vb, gb, True, rows, keys, bf16=True,
                                                       round_o=round_o)
        _assert_grad_close(dq[:, rows], rq, f"{name} dq ({rows.size} rows, round_o={round_o})")
        _assert_grad_close(dk[:, keys], rk, f"{name} dk ({keys.size} keys, round_o={round_o})")
        _assert_grad_close(dv[:, keys], rv, f"{name} dv ({keys.size} keys, round_o={round_o})")
    # identities over every key.  A wrong or dropped term (delta, a sign, the log-sum-exp)
    # moves these sums by the order of the root-sum-square (rss) of the summed elements; the
    # bf16 roundings (2^-9 per output element, per weight and dS, and in each row's
    # normalisation through the log-sum-exp) accumulated over tens of thousands of keys and
    # rows stay at a few percent of it (measured about 1 %).  32 * 2^-9 (6 %) separates the two.
    g = synth.bf16_bits_to_f32(gb).astype(np.float64).reshape(1, S, Hkv, Hq // Hkv, 128)
    want_v = g.sum(axis=(1, 3))
    got_v, got_k = dv.sum(axis=1), dk.sum(axis=1)
    rss_v, rss_k = np.sqrt((dv ** 2).sum(axis=1)), np.sqrt((dk ** 2).sum(axis=1))
    err_v = np.abs(got_v - want_v) / rss_v
    err_k = np.abs(got_k) / rss_k
    print(f"{name}: sum dV vs sum dO {err_v.max():.3e}, sum dK {err_k.max():.3e} (of the rss)", flush=True)
    assert err_v.max() <= 32 * 2.0 ** -9, f"{name}: sum of dV off by {err_v.max():.3e} of its rss"
    assert err_k.max() <= 32 * 2.0 ** -9, f"{name}: sum of dK off by {err_k.max():.3e} of its rss"
