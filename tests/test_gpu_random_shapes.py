"""Seeded random shapes through every launch form the sizes select, against the oracle.

The forward picks 256-row, 128-row (key split) or 64-row (chain split) blocks,
paired or not, from the grid's size; the split forward cuts long blocks into
units where its schedule model says so; the gradients run dQ and dK/dV in one
ordered launch or in two.  These cases draw batch, length, head counts, grouping
and mask from a fixed seed (lengths up to 3000, so that the oracle compares
every element), and check the plain forward with its log-sum-exp, the split
forward, and the gradients at the usual bars (bf16 forward max-abs 1e-2 /
mean-abs 1e-3, lse 2.5e-3; gradients 1 % of the largest and 0.5 % of the mean
magnitude).  Each case prints its shape first.
"""
import numpy as np
import pytest
import torch

import oracle
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
    torch.cuda.synchronize()
    ref = oracle.attention_backward(qb, kb, vb, gb, causal, bf16=True, round_o=True)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        got = host_f64(got)
        assert np.isfinite(got).all(), f"{name} {case}"
        err = np.abs(got - want)
        big, avg = np.abs(want).max(initial=0.0), np.abs(want).mean() if want.size else 0.0
        print(f"  {name}: max {err.max(initial=0.0):.3e} of {big:.3e}", flush=True)
        assert err.max(initial=0.0) <= MAX_REL * big + 1e-6, f"{name} {case}"
        assert (err.mean() if err.size else 0.0) <= MEAN_REL * avg + 1e-7, f"{name} {case}"
