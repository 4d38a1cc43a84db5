"""Seeded random shapes through every launch form the sizes select, against the oracle.

The forward picks 256-row, 128-row (key split) or 64-row (chain split) blocks,
paired or not, from the grid's size; the split forward cuts long blocks into
units where its schedule model says so; the gradients run dQ and dK/dV in one
ordered launch or in two.  These cases draw batch, length, head counts, grouping
and mask from a fixed seed (lengths up to 3000, so that the oracle compares
every element), and check the plain forward with its log-sum-exp, the split
forward, and the gradients at the usual bars (bf16 forward max-abs 1e-2 /
mean-abs 1e-3, lse 2.5e-3; gradients 1 % of the largest and 0.5 % of the mean
magnitude), the gradients also through the split call (the longest dK/dV blocks on
several workgroups where its plan says so).  Key/value chunk visits get the same treatment: seeded query and
key lengths and global offsets (so that the causal diagonal falls anywhere, or
nowhere), a first visit, a second visit merged in the same launch, and the
first visit's gradient contributions from the merged result.  Each case
prints its shape first.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import chunk as ochunk
from helpers import assert_bf16_close, dev_bf16, host_f64
from sequence_long_context_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sequence_long_context_amd import ulysses as U

LSE_ABS = 2.5e-3
MAX_REL, MEAN_REL = 1e-2, 5e-3


def _shapes(seed, n, max_s):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(g.choice([1, 1, 2, 3]))
        S = int(g.integers(1, max_s + 1))
        Hkv = int(g.choice([1, 2, 4]))
        Hq = Hkv * int(g.choice([1, 2, 4]))
        out.append((B, S, Hq, Hkv, bool(g.integers(0, 2))))
    return out


FWD = _shapes(20251203, 12, 3000)
BWD = _shapes(20251204, 8, 1500)


def _chunk_cases(seed, n):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(g.choice([1, 2]))
        Hkv = int(g.choice([1, 2]))
        Hq = Hkv * int(g.choice([1, 2, 4]))
        Sq, Skv = int(g.integers(1, 1200)), int(g.integers(1, 1200))
        k0 = int(g.integers(0, 3000))
        q0 = int(max(0, k0 + g.integers(-Sq, Skv + Sq)))
        out.append((B, Sq, Skv, Hq, Hkv, bool(g.integers(0, 2)), q0, k0))
    return out


CHUNKS = _chunk_cases(20251205, 8)


def _inputs(case, with_dout=False):
    B, S, Hq, Hkv, _ = case
    seed = 97 * S + 13 * Hq + 5 * Hkv + B
    q = synth.normal(seed, (B, S, Hq, 128))
    k = synth.normal(seed + 1, (B, S, Hkv, 128))
    v = synth.normal(seed + 2, (B, S, Hkv, 128))
    return (q, k, v, synth.normal(seed + 3, (B, S, Hq, 128))) if with_dout else (q, k, v)


@pytest.mark.parametrize("case", FWD, ids=[f"B{b}-S{s}-q{hq}-kv{hk}-{'c' if c else 'n'}"
                                          for b, s, hq, hk, c in FWD])
def test_random_forward(case):
    B, S, Hq, Hkv, causal = case
    print(f"random forward B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    qb, kb, vb = _inputs(case)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
    U.ulysses_attention_local_lse(q, k, v, o, lse, causal)
    nbytes = U.ulysses_attention_local_split_workspace(B, S, Hq, causal)
    ws = torch.empty((nbytes // 4,), device="cuda") if nbytes else None
    o_split = torch.empty_like(q)
    lse_split = torch.empty_like(lse)
    U.ulysses_attention_local_split(q, k, v, o_split, causal, ws, lse_split)
    torch.cuda.synchronize()
    print(f"  split workspace {nbytes} bytes", flush=True)
    want = oracle.attention(qb, kb, vb, causal, bf16=True)
    edge = S < 256
    assert_bf16_close(host_f64(o), want, f"forward {case}", edge=edge)
    assert_bf16_close(host_f64(o_split), want, f"split forward {case}", edge=edge)
    ref_lse = oracle.attention_backward(qb, kb, vb, np.zeros_like(qb), causal, bf16=True)[3]
    for name, got in (("lse", lse), ("split lse", lse_split)):
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref_lse).max()
        assert err <= LSE_ABS, f"{name} {case}: {err:.3e}"


@pytest.mark.parametrize("case", BWD, ids=[f"B{b}-S{s}-q{hq}-kv{hk}-{'c' if c else 'n'}"
                                          for b, s, hq, hk, c in BWD])
def test_random_gradients(case):
    B, S, Hq, Hkv, causal = case
    print(f"random gradients B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    qb, kb, vb, gb = _inputs(case, with_dout=True)
    q, k, v, g = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
    U.ulysses_attention_local_lse(q, k, v, o, lse, causal)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    U.ulysses_attention_local_backward(q, k, v, o, g, lse, delta, dq, dk, dv, causal)
    nbytes = U.ulysses_attention_local_backward_split_workspace(B, S, Hq, Hkv, causal)
    ws = torch.empty((nbytes // 4,), device="cuda") if nbytes else None
    sq, sk, sv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    U.ulysses_attention_local_backward_split(q, k, v, o, g, lse, delta, sq, sk, sv, causal, ws)
    torch.cuda.synchronize()
    print(f"  split gradients workspace {nbytes} bytes", flush=True)
    ref = oracle.attention_backward(qb, kb, vb, gb, causal, bf16=True, round_o=True)
    for name, got, want in zip(("dq", "dk", "dv", "split dq", "split dk", "split dv"),
                               (dq, dk, dv, sq, sk, sv), ref[:3] * 2):
        got = host_f64(got)
        assert np.isfinite(got).all(), f"{name} {case}"
        err = np.abs(got - want)
        big, avg = np.abs(want).max(initial=0.0), np.abs(want).mean() if want.size else 0.0
        print(f"  {name}: max {err.max(initial=0.0):.3e} of {big:.3e}", flush=True)
        assert err.max(initial=0.0) <= MAX_REL * big + 1e-6, f"{name} {case}"
        assert (err.mean() if err.size else 0.0) <= MEAN_REL * avg + 1e-7, f"{name} {case}"


def _grad_close(got, want, what):
    assert np.isfinite(got).all(), what
    err = np.abs(got - want)
    big, avg = np.abs(want).max(initial=0.0), np.abs(want).mean() if want.size else 0.0
    print(f"  {what}: max {err.max(initial=0.0):.3e} of {big:.3e}", flush=True)
    assert err.max(initial=0.0) <= MAX_REL * big + 1e-6, what
    assert (err.mean() if err.size else 0.0) <= MEAN_REL * avg + 1e-7, what


def _check_visit(got_o, got_l, want_o, want_l, what):
    empty = np.isneginf(want_l)  # [B][Hq][Sq]
    assert np.array_equal(np.isneginf(got_l), empty), f"{what}: rows without a visible key differ"
    e_rows = np.transpose(empty, (0, 2, 1))
    assert np.all(got_o[e_rows] == 0.0), f"{what}: rows without a visible key must be 0"
    if (~e_rows).any():
        assert_bf16_close(got_o[~e_rows], want_o[~e_rows], what, edge=True)
        err = np.abs(got_l[~empty] - want_l[~empty]).max()
        assert err <= LSE_ABS, f"{what} lse: {err:.3e}"


@pytest.mark.parametrize("case", CHUNKS, ids=[f"B{b}-q{sq}-k{sk}-h{hq}-{hk}-{'c' if c else 'n'}-{q0}-{k0}"
                                              for b, sq, sk, hq, hk, c, q0, k0 in CHUNKS])
def test_random_chunk_visits(case):
    B, Sq, Skv, Hq, Hkv, causal, q0, k0 = case
    print(f"random chunk B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv} causal={causal} "
          f"q_pos0={q0} k_pos0={k0}", flush=True)
    seed = 31 * Sq + 17 * Skv + 7 * q0 + k0
    qb = synth.normal(seed, (B, Sq, Hq, 128))
    kb, vb, kb2, vb2 = (synth.normal(seed + 1 + i, (B, Skv, Hkv, 128)) for i in range(4))
    q, k, v, k2, v2 = (dev_bf16(x) for x in (qb, kb, vb, kb2, vb2))
    o = torch.full_like(q, float("nan"))  # every element must be written
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda", dtype=torch.float32)
    U.ulysses_attention_chunk(q, k, v, o, lse, causal, q0, k0)
    torch.cuda.synchronize()
    wo, wl = ochunk.attention_chunk(qb, kb, vb, causal, q0, k0, bf16=True)
    _check_visit(host_f64(o), lse.cpu().numpy().astype(np.float64), wo, wl, "first visit")
    # a second chunk, the keys just before the first, merged in the same launch
    k0b = max(0, k0 - Skv)
    U.ulysses_attention_chunk_accumulate(q, k2, v2, o, lse, causal, q0, k0b)
    torch.cuda.synchronize()
    wo2, wl2 = ochunk.attention_chunk(qb, kb2, vb2, causal, q0, k0b, bf16=True)
    mo, ml = ochunk.softmax_merge(wo, wl, wo2, wl2)
    _check_visit(host_f64(o), lse.cpu().numpy().astype(np.float64), mo, ml, "merged visit")
    # the first visit's gradient contributions, from the merged output and lse
    gb = synth.normal(seed + 9, (B, Sq, Hq, 128))
    ob = synth.f32_to_bf16_bits(mo.astype(np.float32))
    lt = torch.from_numpy(ml.astype(np.float32)).cuda()
    delta = torch.empty_like(lt)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    U.ulysses_attention_chunk_backward(q, k, v, dev_bf16(ob), dev_bf16(gb), lt, delta, dq, dk, dv,
                                       causal, q0, k0)
    torch.cuda.synchronize()
    ref = ochunk.attention_chunk_backward(qb, kb, vb, gb, ob, ml, causal, q0, k0, bf16=True)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _grad_close(host_f64(got), want, name)
