"""The path under HIP graph capture.

The library allocates nothing and each call only enqueues kernels on the
caller's stream, so a whole step (the Q, K, V exchange, one rank's attention,
the inverse exchange, and a key/value chunk merged into a running result) can
be captured once and replayed.  Every kernel is deterministic (fixed
reduction order), so each replay must reproduce the eager results bit for
bit; replays are interleaved with eager work and host synchronisation.
The eager results themselves are checked against the oracle by the other
GPU tests; here the chunk visit's output is also compared with the oracle.
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


def _bits(t):
    torch.cuda.synchronize()
    return t.cpu().view(torch.int16).numpy().copy()


def test_step_graph_replays_match_eager():
    B, S, H, D, P = 1, 4096, 32, 128, 8
    hq = H // P
    seq = {t: dev_bf16(synth.normal(500 + i, (P, B, S // P, H, D))) for i, t in enumerate("qkv")}
    head = {t: torch.empty((P, B, S, hq, D), dtype=torch.bfloat16, device="cuda") for t in "qkv"}
    o_head = torch.empty((P, B, S, hq, D), dtype=torch.bfloat16, device="cuda")
    o_seq = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device="cuda")
    # a ring visit on rank 0's heads: the second half's queries against the first half
    h = S // 2
    acc_o = torch.empty((B, S - h, hq, D), dtype=torch.bfloat16, device="cuda")
    acc_l = torch.empty((B, hq, S - h), dtype=torch.float32, device="cuda")

    def step():
        U.ulysses_seq_to_head_qkv(seq["q"], seq["k"], seq["v"], head["q"], head["k"], head["v"], P)
        U.ulysses_attention_local(head["q"][0], head["k"][0], head["v"][0], o_head[0], True)
        U.ulysses_head_to_seq(o_head, o_seq, P)
        qb = head["q"][0][:, h:]
        U.ulysses_attention_chunk(qb.contiguous(), head["k"][0][:, h:].contiguous(),
                                  head["v"][0][:, h:].contiguous(), acc_o, acc_l, True, h, h)
        U.ulysses_attention_chunk_accumulate(qb.contiguous(), head["k"][0][:, :h].contiguous(),
                                             head["v"][0][:, :h].contiguous(), acc_o, acc_l, True, h, 0)

    o_head.zero_()
    step()
    want = {"o_seq": _bits(o_seq), "acc_o": _bits(acc_o), "acc_l": acc_l.cpu().numpy().copy()}

    # the ring visit pair against the oracle (rank 0's heads, rows h.., every key)
    qh = head["q"][0].cpu().view(torch.int16).numpy().view(np.uint16)
    kh = head["k"][0].cpu().view(torch.int16).numpy().view(np.uint16)
    vh = head["v"][0].cpu().view(torch.int16).numpy().view(np.uint16)
    rows = np.arange(h, S, 61)
    w_o = np.stack([oracle.attention_chunk(qh[:, i:i + 1], kh, vh, True, q_pos0=int(i), bf16=True)[0][:, 0]
                    for i in rows], axis=1)
    assert_bf16_close(host_f64(acc_o)[:, rows - h], w_o, "graph test: ring visit pair (eager)")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        o_seq.fill_(0)
        acc_o.fill_(0)
        acc_l.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"graph replay {rep}", flush=True)
        assert np.array_equal(_bits(o_seq), want["o_seq"]), f"replay {rep}: o_seq"
        assert np.array_equal(_bits(acc_o), want["acc_o"]), f"replay {rep}: ring output"
        assert np.array_equal(acc_l.cpu().numpy(), want["acc_l"]), f"replay {rep}: ring lse"
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_gradient_and_split_graph_replays_match_eager():
    """A training-shaped step under capture: the forward with its log-sum-exp and the gradient
    call (S = 4096 with 4 heads, where dQ and dK/dV share one ordered launch whose order
    travels as a kernel argument), the split gradients of the same call (the longest dK/dV
    blocks on several workgroups, fp32 slots in a caller workspace, a summing launch), plus
    the split forward at one head per rank (two launches and a caller workspace).  Three
    replays, with eager work between them, bit for bit equal to the eager results."""
    B, S, H, D = 1, 4096, 4, 128
    q, k, v, g = (dev_bf16(synth.normal(700 + i, (B, S, H, D))) for i in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    q1, k1, v1 = (t[:, :, :1].contiguous() for t in (q, k, v))
    o1 = torch.empty_like(q1)
    nbytes = U.ulysses_attention_local_split_workspace(B, S, 1, True)
    assert nbytes > 0
    ws = torch.empty((nbytes // 4,), dtype=torch.float32, device="cuda")
    bbytes = U.ulysses_attention_local_backward_split_workspace(B, S, H, H, True)
    assert bbytes > 0
    bws = torch.empty((bbytes // 4,), dtype=torch.float32, device="cuda")
    sdq, sdk, sdv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        U.ulysses_attention_local_lse(q, k, v, o, lse, True)
        U.ulysses_attention_local_backward(q, k, v, o, g, lse, delta, dq, dk, dv, True)
        U.ulysses_attention_local_backward_split(q, k, v, o, g, lse, delta, sdq, sdk, sdv, True, bws)
        U.ulysses_attention_local_split(q1, k1, v1, o1, True, ws)

    step()
    outs = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "o1": o1, "sdq": sdq, "sdk": sdk,
            "sdv": sdv}
    want = {n: t.cpu().numpy().copy() if t.dtype == torch.float32 else _bits(t) for n, t in outs.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for rep in range(3):
        for t in outs.values():
            t.fill_(0)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        print(f"gradient graph replay {rep}", flush=True)
        for n, t in outs.items():
            got = t.cpu().numpy() if t.dtype == torch.float32 else _bits(t)
            assert np.array_equal(got, want[n]), f"replay {rep}: {n}"
        step()  # eager work between replays
        torch.cuda.synchronize()
