"""GPU parity of the split forward (ulysses_attention_local_split) against the oracle.

The key tiles of each 64-row query block may be cut into ranges handled by
different workgroups, whose partial results are merged by their share of the
exp-sum.  Outputs must meet the forward's bars against the fp64 oracle (bf16:
max-abs 1e-2, mean-abs 1e-3; the edge-case bars for a handful of keys), and
lse the 2.5e-3 bar of the bf16 row sums.  The shapes cover sizes whose plan
splits blocks (short sequences, causal and not, grouped heads, ragged last
blocks, several batch entries) and sizes where nothing is split (the call is
then the plain one and needs no workspace); each case prints whether the plan
split it.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_bf16_close, dev_bf16, host_f64, stratified_rows
from sequence_long_context_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sequence_long_context_amd import ulysses as U

LSE_ABS = 2.5e-3


def _split_gpu(q, k, v, causal):
    B, S, Hq, _ = q.shape
    nbytes = U.ulysses_attention_local_split_workspace(B, S, Hq, causal)
    ws = torch.zeros((max(nbytes, 16) // 4,), device="cuda") if nbytes else None
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
    U.ulysses_attention_local_split(q, k, v, o, causal, ws, lse)
    o2 = torch.empty_like(q)  # without lse, and a second call on the same workspace
    U.ulysses_attention_local_split(q, k, v, o2, causal, ws)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "repeated call or lse changes o"
    return o, lse, nbytes


@pytest.mark.parametrize("B,S,Hq,Hkv,causal", [
    (1, 4096, 1, 1, True), (1, 4096, 1, 1, False), (1, 4096, 2, 1, True), (2, 3000, 1, 1, True),
    (1, 3000, 1, 1, True), (1, 4096, 4, 4, True), (1, 300, 2, 2, True), (1, 65, 1, 1, True),
    (1, 1, 1, 1, True), (3, 200, 4, 2, False)])
def test_split_forward(B, S, Hq, Hkv, causal):
    print(f"split forward B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    seed = 31 * S + 7 * Hq + B
    qb = synth.normal(seed, (B, S, Hq, 128))
    kb = synth.normal(seed + 1, (B, S, Hkv, 128))
    vb = synth.normal(seed + 2, (B, S, Hkv, 128))
    o, lse, nbytes = _split_gpu(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), causal)
    print(f"  workspace {nbytes} bytes ({'split' if nbytes else 'not split'})", flush=True)
    want = oracle.attention(qb, kb, vb, causal, bf16=True)
    assert_bf16_close(host_f64(o), want, f"split B={B} S={S} causal={causal}", edge=S < 256)
    ref_lse = oracle.attention_backward(qb, kb, vb, np.zeros_like(qb), causal, bf16=True)[3]
    err = np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse).max()
    print(f"  lse max err {err:.2e}", flush=True)
    assert err <= LSE_ABS


def test_split_long_sampled():
    """S = 8192 with 1 head (split into about 260 units), on 1024 stratified rows
    of the oracle."""
    B, S, H = 1, 8192, 1
    qb, kb, vb = (synth.normal(900 + i, (B, S, H, 128)) for i in range(3))
    o, _, nbytes = _split_gpu(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), True)
    assert nbytes > 0
    rows = stratified_rows(S, 8, 1024, 5)
    want = oracle.attention(qb, kb, vb, True, bf16=True, rows=rows)
    assert_bf16_close(host_f64(o)[:, rows], want, "split S=8192 sampled")


def test_split_workspace_and_errors():
    need = U.ulysses_attention_local_split_workspace(1, 4096, 1, True)
    assert need > 0
    # query blocks that balance the GPU by themselves: nothing split, no workspace
    assert U.ulysses_attention_local_split_workspace(1, 65536, 4, True) == 0
    assert U.ulysses_attention_local_split_workspace(1, 32768, 4, True) == 0
    q = torch.zeros((1, 4096, 1, 128), device="cuda", dtype=torch.bfloat16)
    o = torch.empty_like(q)
    small = torch.empty(((need - 16) // 4,), device="cuda")
    with pytest.raises(U.UlyssesError, match="workspace") as err:
        U.ulysses_attention_local_split(q, q, q, o, True, small)
    assert err.value.status == U.ULY_ERR_INVALID_ARGUMENT
    with pytest.raises(U.UlyssesError, match="workspace"):
        U.ulysses_attention_local_split(q, q, q, o, True, None)


def test_split_matches_plain_call():
    """Against the plain call at the 4k workload's length with 2 heads per rank
    (S = 4096, causal): the same attention to rounding; equal bits where the plan
    splits nothing."""
    S, H = 4096, 2
    qb, kb, vb = (synth.normal(synth.seed_for(1, t), (1, S, H, 128)) for t in "qkv")
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    ws = torch.zeros((U.ulysses_attention_local_split_workspace(1, S, H, True) // 4,), device="cuda")
    o1, op = torch.empty_like(q), torch.empty_like(q)
    U.ulysses_attention_local_split(q, k, v, o1, True, ws)
    U.ulysses_attention_local(q, k, v, op, True)
    torch.cuda.synchronize()
    d = (o1.float() - op.float()).abs()
    print(f"split vs plain: max {d.max().item():.3e} mean {d.mean().item():.3e}", flush=True)
    assert d.max().item() <= 2e-2 and d.mean().item() <= 1e-3
    # nothing split: the plain call itself
    q2 = q[:, :256].contiguous()
    assert U.ulysses_attention_local_split_workspace(1, 256, H, True) == 0
    o2, o3 = torch.empty_like(q2), torch.empty_like(q2)
    U.ulysses_attention_local_split(q2, q2, q2, o2, True)
    U.ulysses_attention_local(q2, q2, q2, o3, True)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o3.view(torch.int16))
