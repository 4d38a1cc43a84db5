"""GPU parity of the split gradients (ulysses_attention_local_backward_split).

The longest dK/dV key blocks' query streams are cut into units on several
workgroups, whose fp32 sums meet in the workspace and are added in unit order
by the block's last unit.  Checked on sizes whose plan cuts blocks (the short
workload's rank shape S = 4096 with 4 heads, both masks; grouped heads; ragged
lengths; several batch entries) and on sizes where nothing is cut (the call is
then the plain one): dq, dk, dv against the fp64 oracle at the gradient bars
(max error 1 % of the largest, mean error 0.5 % of the mean magnitude), dq
equal bit for bit to the plain call's, dk and dv equal to it up to the order of
the fp32 sums, and a second call on the same workspace equal bit for bit to
the first.  Each case prints whether the plan cut it.
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

MAX_REL, MEAN_REL = 1e-2, 5e-3


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("B,S,Hq,Hkv,causal", [
    (1, 4096, 4, 4, True), (1, 4096, 4, 4, False), (1, 2048, 4, 1, True), (2, 3000, 2, 2, True),
    (1, 1500, 8, 2, False), (1, 700, 2, 1, True), (1, 200, 1, 1, True)])
def test_split_gradients(B, S, Hq, Hkv, causal):
    print(f"split gradients B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    seed = 41 * S + 7 * Hq + 3 * Hkv + B
    qb, gb = synth.normal(seed, (B, S, Hq, 128)), synth.normal(seed + 3, (B, S, Hq, 128))
    kb, vb = synth.normal(seed + 1, (B, S, Hkv, 128)), synth.normal(seed + 2, (B, S, Hkv, 128))
    q, k, v, g = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
    U.ulysses_attention_local_lse(q, k, v, o, lse, causal)
    delta = torch.empty_like(lse)
    nbytes = U.ulysses_attention_local_backward_split_workspace(B, S, Hq, Hkv, causal)
    print(f"  workspace {nbytes} bytes ({'split' if nbytes else 'not split'})", flush=True)
    ws = torch.empty((nbytes // 4,), device="cuda") if nbytes else None
    runs = []
    for _ in range(2):  # the second call on the same workspace
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        U.ulysses_attention_local_backward_split(q, k, v, o, g, lse, delta, dq, dk, dv, causal, ws)
        runs.append((dq, dk, dv))
    pq, pk, pv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    U.ulysses_attention_local_backward(q, k, v, o, g, lse, delta, pq, pk, pv, causal)
    torch.cuda.synchronize()
    for a, b, name in zip(runs[0], runs[1], ("dq", "dk", "dv")):
        assert _same(a, b), f"{name}: a second call on the same workspace differs"
    dq, dk, dv = runs[0]
    assert _same(dq, pq), "dq differs from the plain call"
    for got, plain, name in ((dk, pk, "dk"), (dv, pv, "dv")):
        d = (got.float() - plain.float()).abs().max().item()
        big = plain.float().abs().max().item()
        print(f"  {name} vs plain call: max {d:.3e} of {big:.3e}", flush=True)
        assert d <= 1e-2 * big + 1e-6, name
        if not nbytes:
            assert _same(got, plain), f"{name}: nothing split, yet not the plain call's bits"
    ref = oracle.attention_backward(qb, kb, vb, gb, causal, bf16=True, round_o=True)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        got = host_f64(got)
        assert np.isfinite(got).all(), name
        err = np.abs(got - want)
        big, avg = np.abs(want).max(initial=0.0), np.abs(want).mean()
        print(f"  {name}: max {err.max():.3e} of {big:.3e}, mean {err.mean():.3e} of {avg:.3e}", flush=True)
        assert err.max() <= MAX_REL * big + 1e-6, name
        assert err.mean() <= MEAN_REL * avg + 1e-7, name


def test_split_gradients_workspace_errors():
    need = U.ulysses_attention_local_backward_split_workspace(1, 4096, 4, 4, True)
    assert need > 0
    # 256-row dQ blocks (long sequences): the plain two launches, nothing split
    assert U.ulysses_attention_local_backward_split_workspace(1, 32768, 4, 4, True) == 0
    q = torch.zeros((1, 4096, 4, 128), device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros((1, 4, 4096), device="cuda")
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    small = torch.empty(((need - 256) // 4,), device="cuda")
    for ws in (small, None):
        with pytest.raises(U.UlyssesError, match="workspace") as err:
            U.ulysses_attention_local_backward_split(q, q, q, q, q, lse, delta, dq, dk, dv, True, ws)
        assert err.value.status == U.ULY_ERR_INVALID_ARGUMENT
