"""The allocation-free gradient call (ulysses_attention_local_backward_noalloc)
against the call that takes a delta workspace (ulysses_attention_local_backward),
through the C ABI: calls in a row on one GPU, the first filling the scratch,
each later one smaller (so the scratch holds the larger contents of the call
before when it starts), each bit for bit equal to the workspace call on the
same inputs (the same kernels, with delta in the library's scratch).  Also: a size
beyond the scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

from helpers import dev_bf16
from sequence_long_context_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sequence_long_context_amd import ulysses as U


def _inputs(seed, B, S, Hq, Hkv, causal):
    q, g = (dev_bf16(synth.normal(seed + i, (B, S, Hq, 128))) for i in (0, 3))
    k, v = (dev_bf16(synth.normal(seed + i, (B, S, Hkv, 128))) for i in (1, 2))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
    U.ulysses_attention_local_lse(q, k, v, o, lse, causal)
    return q, k, v, o, g, lse


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def test_noalloc_matches_workspace_call_in_a_row():
    # the first call fills the scratch exactly (B * Hq * S = 2^20); each later one is smaller
    cases = [(1, 131072, 8, 2, True, 3), (2, 3000, 8, 2, True, 1), (1, 777, 4, 4, False, 2)]
    for B, S, Hq, Hkv, causal, seed in cases:
        print(f"noalloc gradients B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
        q, k, v, o, g, lse = _inputs(100 * seed, B, S, Hq, Hkv, causal)
        ref = [torch.empty_like(x) for x in (q, k, v)]
        delta = torch.empty_like(lse)
        U.ulysses_attention_local_backward(q, k, v, o, g, lse, delta, *ref, causal)
        got = [torch.full_like(x, float("nan")) for x in (q, k, v)]
        U.ulysses_attention_local_backward_noalloc(q, k, v, o, g, lse, *got, causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert np.array_equal(_bits(a), _bits(b)), f"{name} differs from the workspace call"
            assert torch.isfinite(a.float()).all()


def test_noalloc_refuses_sizes_beyond_the_scratch():
    # real buffers of the refused size, so that every other check passes
    B, S, Hq, Hkv = 1, 262145, 4, 4  # B * Hq * S = 2^20 + 4
    q, k, v, o, g = (torch.zeros((B, S, h, 128), device="cuda", dtype=torch.bfloat16)
                     for h in (Hq, Hkv, Hkv, Hq, Hq))
    lse = torch.zeros((B, Hq, S), device="cuda", dtype=torch.float32)
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    with pytest.raises(U.UlyssesError, match="scratch") as err:
        U.ulysses_attention_local_backward_noalloc(q, k, v, o, g, lse, dq, dk, dv, True)
    assert err.value.status == U.ULY_ERR_UNSUPPORTED
