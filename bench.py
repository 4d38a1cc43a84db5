"""Benchmark of the Ulysses attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input, with P virtual
ranks in one HBM: seq->head of Q, K and V (all P shards), one rank's
full-sequence attention on its heads, head->seq of the attention output (all
P shards).  Inputs are resident in HBM before the timed region.

Default workload (s32k): B=1, S=32768, 32 heads x head_dim 128 (hidden 4096),
P=8 -> 4 heads per rank, bf16, causal.  Prints one JSON line:
  value            attention TFLOP/s (4*D flops per visible query/key pair)
  transpose        layout-change GB/s (one read + one write per element); also
                   Q, K, V seq->head in one launch (timed after the steps)
  roofline         the attention kernel against the bf16 MFMA peak
  roofline_layout  the layout kernel against the HBM peak
  cpu_baseline     the fp64 CPU oracle on a bounded sample of the same workload
  backward         (bf16 only, not part of `value`) the gradients of the same
                   rank's attention: delta + dQ + dK/dV kernels, timed after the
                   steps; algorithmic flops 2.5x the forward's (five S x S x D
                   products: Q K^T, dO V^T, P^T dO, dS^T Q, dS K)
  ring             (bf16) the rank's sequence split over a ring of degree 2
  pieces           (bf16) the rank's tokens as two batch entries: the attention
                   reading and writing the exchange's piece order against the
                   plain attention, and the unpack / pack passes it removes
Kernel durations come from HIP events recorded on the stream the kernels run on
(5 warmup steps, 50 timed by default).  The transposes read one of three
identical input sets per step, so no input is still cached from the previous
step (three sets exceed the 256 MiB MALL); `transpose.frac_memcpy` compares their
rate with a device-to-device copy of the same bytes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBPS = 8000.0
# exponentials per second: 256 CUs x 4 SIMDs x 8 lanes per clock (a wave64
# v_exp_f32 issues every 8 cycles on gfx950) x 2.4 GHz
PEAK_EXP_PER_S = 256 * 4 * 8 * 2.4e9
NSETS = 3  # input buffer sets the transposes rotate through (more than the 256 MiB MALL holds)

WORKLOADS = {
    # name: (seed id, B, S, Hq, Hkv, D, P, dtype, causal)
    "tiny": (0, 1, 256, 4, 4, 32, 4, "f32", False),
    "s4k": (1, 1, 4096, 32, 32, 128, 8, "bf16", True),
    "s32k": (2, 1, 32768, 32, 32, 128, 8, "bf16", True),
    "s64k_gqa": (3, 1, 65536, 32, 8, 128, 8, "bf16", True),
    "s256k": (4, 1, 262144, 32, 32, 128, 32, "bf16", True),
}


def measured_traffic(summary, sources, directory=None):
    """HBM bytes per launch recorded by a counter summary under profiles/, or None.

    The summary names the SHA-256 of each kernel source it was taken from; a
    source that has changed since makes the figure stale, and None is returned.
    Lines read: 'source <relative path> sha256 <hex>' and
    'hbm_bytes_per_launch <workload> <integer>'."""
    import hashlib
    path = os.path.join(directory or os.path.join(ROOT, "profiles"), summary)
    if not os.path.exists(path):
        return {}
    want, out = {}, {}
    for line in open(path):
        f = line.split()
        if len(f) == 4 and f[0] == "source" and f[2] == "sha256":
            want[f[1]] = f[3]
        elif len(f) == 3 and f[0] == "hbm_bytes_per_launch":
            out[f[1]] = int(f[2])
    for src in sources:
        full = os.path.join(ROOT, src)
        if src not in want or not os.path.exists(full):
            return {}
        if hashlib.sha256(open(full, "rb").read()).hexdigest() != want[src]:
            return {}
    return out


ATTN_SOURCES = ["sequence_long_context_amd/csrc/attn_fwd.h",
                "sequence_long_context_amd/csrc/attention_bf16.hip",
                "sequence_long_context_amd/csrc/attn_tiles.h",
                "sequence_long_context_amd/csrc/api.hip"]
LAYOUT_SOURCES = ["sequence_long_context_amd/csrc/layout.hip",
                  "sequence_long_context_amd/csrc/api.hip"]


def attention_flops(S, hq, D, causal, rows=None):
    """4*D flops (QK^T and PV, multiply+add) per visible (query, key) pair."""
    if rows is None:
        pairs = S * (S + 1) // 2 if causal else S * S
    else:
        rows = np.asarray(rows, dtype=np.int64)
        pairs = int((rows + 1).sum()) if causal else S * rows.size
    return 4.0 * D * hq * pairs


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="s32k", choices=sorted(WORKLOADS))
    ap.add_argument("--rank", type=int, default=0, help="virtual rank whose attention is timed")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after timing, run one plain 256 MiB device copy (for counter calibration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the gradient timing")
    ap.add_argument("--no-ring", action="store_true", help="skip the key/value-chunk timing")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the one-head-per-rank timing of the split forward")
    ap.add_argument("--no-pieces", action="store_true",
                    help="skip the timing of the attention in the exchange's piece order")
    ap.add_argument("--cpu-row-stride", type=int, default=0,
                    help="CPU baseline: every n-th query row of the timed rank, all its heads "
                         "(0: every row when that is estimated under ~30 s, else the smallest "
                         "power of two that is)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the P ranks are simulated inside one GPU's HBM", file=sys.stderr)
        sys.exit(2)

    import torch
    from sequence_long_context_amd import synth
    from sequence_long_context_amd import ulysses as U

    wid, B, S, Hq, Hkv, D, P, dt, causal = WORKLOADS[args.workload]
    hq, hkv = Hq // P, Hkv // P
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32

    def upload(a):
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    host = {}
    sets = [{} for _ in range(NSETS)]
    for t, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        a = synth.normal(synth.seed_for(wid, t), (P, B, S // P, H, D), dt)
        host[t] = a
        sets[0][t] = upload(a)
        for k in range(1, NSETS):  # identical copies: step i reads set i % NSETS
            sets[k][t] = sets[0][t].clone()
    heads = {t: torch.empty((P, B, S, (Hq if t == "q" else Hkv) // P, D), dtype=tdt, device=dev)
             for t in "qkv"}
    o_head = torch.zeros((P, B, S, hq, D), dtype=tdt, device=dev)
    o_seq = torch.empty((P, B, S // P, Hq, D), dtype=tdt, device=dev)
    r = args.rank

    # one step: the seq->head exchange of Q, K and V in one launch, rank r's
    # attention, the head->seq exchange of O
    def step(ev=None, i=0):
        seqs = sets[i % NSETS]
        if ev: ev[0].record()
        U.ulysses_seq_to_head_qkv(seqs["q"], seqs["k"], seqs["v"], heads["q"], heads["k"], heads["v"], P)
        if ev: ev[1].record()
        U.ulysses_attention_local(heads["q"][r], heads["k"][r], heads["v"][r], o_head[r], causal)
        if ev: ev[2].record()
        U.ulysses_head_to_seq(o_head, o_seq, P)
        if ev: ev[3].record()

    for i in range(args.warmup):
        step(None, i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i], i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    seg = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(3)]
                    for i in range(args.steps)])  # ms: Q/K/V exchange, attention, O exchange
    step_ms = np.array([evs[i][0].elapsed_time(evs[i][3]) for i in range(args.steps)])
    total_ms = evs[0][0].elapsed_time(evs[-1][3])
    ms_per_step = max(total_ms, wall * 1e3) / args.steps
    t_attn = float(seg[:, 1].mean()) * 1e-3
    lay = seg[:, [0, 2]]
    esz = 2 if dt == "bf16" else 4
    tensor_bytes = {t: 2.0 * B * S * H * D * esz for t, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("o", Hq))}
    lay_bytes = np.array([tensor_bytes["q"] + tensor_bytes["k"] + tensor_bytes["v"], tensor_bytes["o"]])
    lay_gbps = lay_bytes / (lay.mean(axis=0) * 1e-3) / 1e9
    lay_total_gbps = lay_bytes.sum() / (lay.mean(axis=0).sum() * 1e-3) / 1e9
    flops = attention_flops(S, hq, D, causal)
    tflops = flops / t_attn / 1e12
    exps = flops / (4.0 * D)  # one exponential per visible (query, key) pair

    # a device-to-device copy of the same bytes as one Q transpose, for reference
    cp_src = sets[1]["q"].view(-1)
    cp_dst = torch.empty_like(cp_src)
    for _ in range(3):
        cp_dst.copy_(cp_src)
    cp_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cp_ms = []
    for _ in range(10):
        cp_ev[0].record()
        cp_dst.copy_(cp_src)
        cp_ev[1].record()
        torch.cuda.synchronize()
        cp_ms.append(cp_ev[0].elapsed_time(cp_ev[1]))
    memcpy_gbps = 2.0 * cp_src.numel() * cp_src.element_size() / (float(np.median(cp_ms)) * 1e-3) / 1e9
    del cp_dst

    # the same step with Q, K and V exchanged by three separate launches, outside
    # the timed steps, same input rotation: each tensor's exchange on its own
    def step_three(ev, i):
        x = sets[i % NSETS]
        ev[0].record()
        for j, t in enumerate("qkv"):
            U.ulysses_seq_to_head(x[t], heads[t], P)
            ev[j + 1].record()
        U.ulysses_attention_local(heads["q"][r], heads["k"][r], heads["v"][r], o_head[r], causal)
        U.ulysses_head_to_seq(o_head, o_seq, P)
        ev[4].record()
    nq = min(args.steps, 20)
    for i in range(2):
        step_three([torch.cuda.Event(enable_timing=True) for _ in range(5)], i)
    q3 = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(nq)]
    torch.cuda.synchronize()
    for i in range(nq):
        step_three(q3[i], i)
    torch.cuda.synchronize()
    three = np.array([[q3[i][j].elapsed_time(q3[i][j + 1]) for j in range(3)] for i in range(nq)])  # ms
    three_us = np.median(three, axis=0) * 1e3
    three_step_ms = float(np.median([q3[i][0].elapsed_time(q3[i][4]) for i in range(nq)]))

    # the dominant layout launch (the Q/K/V exchange) for the layout roofline
    qkv_lay_s = float(lay[:, 0].mean()) * 1e-3
    qkv_lay_gbps = lay_bytes[0] / qkv_lay_s / 1e9

    out = {
        "metric": "attention TFLOP/s (% bf16 MFMA peak) + transpose GB/s (% HBM) at S=32k",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == "bf16" else "f32",
        "data": "synthetic: seeded N(0,1) Q/K/V",
        "config": {
            "workload": f"{args.workload}: B={B} S={S} heads={Hq} kv_heads={Hkv} head_dim={D} "
                        f"P={P} ({hq} q / {hkv} kv heads per rank) {dt} "
                        f"{'causal' if causal else 'non-causal'}; layout change of all {P} "
                        f"shards of Q, K, V and O, attention of rank {r}",
            "B": B, "S": S, "n_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "P": P,
            "causal": causal,
        },
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4),
            "traffic": measured_traffic("attention_bf16_counters.md", ATTN_SOURCES).get(
                args.workload) if dt == "bf16" else None,
            "kernel": "attention_bf16_d128_kernel" if dt == "bf16" else "attention_f32_kernel",
            "flops_per_launch": flops, "avg_launch_us": round(t_attn * 1e6, 2),
        },
        # the secondary bound of the softmax: its exponentials on the transcendental unit
        "roofline_softmax_exp": {
            "bound": "transcendental", "achieved": round(exps / t_attn, 1), "peak": PEAK_EXP_PER_S,
            "unit": "exp/s", "frac": round(exps / t_attn / PEAK_EXP_PER_S, 4),
            "exps_per_launch": exps,
        },
        "roofline_layout": {
            "bound": "hbm", "achieved": round(qkv_lay_gbps, 1), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(qkv_lay_gbps / PEAK_HBM_GBPS, 4),
            "traffic": measured_traffic("layout_counters.md", LAYOUT_SOURCES).get(args.workload),
            "kernel": "layout3_kernel (seq->head of Q, K and V in one launch)",
            "bytes_per_launch": lay_bytes[0], "avg_launch_us": round(qkv_lay_s * 1e6, 2),
        },
        "transpose": {
            "GB/s": round(lay_total_gbps, 1), "frac_hbm": round(lay_total_gbps / PEAK_HBM_GBPS, 4),
            "memcpy_GB/s": round(memcpy_gbps, 1),
            "frac_memcpy": round(lay_total_gbps / memcpy_gbps, 4),
            "input_sets": NSETS,
            "per_launch_GB/s": {"qkv_s2h": round(lay_gbps[0], 1), "o_h2s": round(lay_gbps[1], 1)},
            "per_launch_us": {"qkv_s2h": round(lay.mean(axis=0)[0] * 1e3, 2),
                              "o_h2s": round(lay.mean(axis=0)[1] * 1e3, 2)},
            "three_launches": {
                "us": {t: round(float(three_us[j]), 2) for j, t in enumerate("qkv")},
                "GB/s": {t: round(tensor_bytes[t] / (three_us[j] * 1e-6) / 1e9, 1)
                         for j, t in enumerate("qkv")},
                "sum_us": round(float(three_us.sum()), 2), "step_ms": round(three_step_ms, 4),
                "timing": "Q, K and V exchanged by separate launches in an untimed copy of the "
                          "step; medians over 20 steps"},
        },
        "attention": {"TFLOP/s": round(tflops, 2), "us": round(t_attn * 1e6, 2),
                      "us_median": round(float(np.median(seg[:, 1])) * 1e3, 2),
                      "us_min": round(float(seg[:, 1].min()) * 1e3, 2), "flops": flops},
        "step_ms_median": round(float(np.median(step_ms)), 4),
    }

    if dt == "bf16" and not args.no_backward:
        out["backward"] = time_backward(U, torch, heads, r, causal, flops, wid, dev)

    if dt == "bf16" and not args.no_ring:
        out["ring"] = time_ring(U, torch, heads, r, causal, dev)

    if dt == "bf16" and not args.no_pieces and (S // 2) % (64 * P) == 0:
        out["pieces"] = time_pieces(U, torch, S, hq, hkv, D, P, causal, wid, dev)

    if dt == "bf16" and not args.no_split:
        out["split"] = time_split(U, torch, heads, r, causal, dev)

    if args.calibration_copy:  # outside the timed region: a plain copy of known size
        src = torch.ones(128 << 20, dtype=torch.bfloat16, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(host, B, S, Hq, Hkv, D, P, hq, hkv, r, dt, causal,
                                           args.cpu_row_stride, args.workload, wid)
    print(json.dumps(out), flush=True)


def time_backward(U, torch, heads, r, causal, fwd_flops, wid, dev, reps=10):
    """Gradients of rank r's attention for a seeded synthetic output gradient, through the
    split call: where its plan cuts the longest dK/dV blocks into units (short sequences,
    grouped heads) with the workspace it asks for, elsewhere the plain call itself."""
    from sequence_long_context_amd import synth
    q, k, v = heads["q"][r], heads["k"][r], heads["v"][r]
    B, S, Hq, D = q.shape
    g = torch.from_numpy(synth.normal(synth.seed_for(wid, "do"), tuple(q.shape)).view(np.int16))
    g = g.view(torch.bfloat16).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    U.ulysses_attention_local_lse(q, k, v, o, lse, causal)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = U.ulysses_attention_local_backward_split_workspace(B, S, Hq, k.shape[2], causal)
    ws = torch.empty((nbytes // 4,), dtype=torch.float32, device=dev) if nbytes else None

    def call():
        U.ulysses_attention_local_backward_split(q, k, v, o, g, lse, delta, dq, dk, dv, causal, ws)
    for _ in range(2):
        call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(reps):
        call()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
    flops = 2.5 * fwd_flops
    tf = flops / (float(ms.mean()) * 1e-3) / 1e12
    finite = bool(torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all()
                  and torch.isfinite(dv.float()).all())
    return {"TFLOP/s": round(tf, 2), "frac": round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
            "us": round(float(ms.mean()) * 1e3, 2), "us_median": round(float(np.median(ms)) * 1e3, 2),
            "flops": flops, "launches": reps, "finite": finite, "split_workspace_bytes": nbytes,
            "kernels": "attention_delta_kernel + attention_bwd_dq_kernel + attention_bwd_dkdv_kernel"
                       + (" (one launch, split dK/dV blocks) + dkdv_split_sum_kernel" if nbytes else "")}


def time_ring(U, torch, heads, r, causal, dev, rounds=4, reps=5):
    """Rank r's sequence split over a ring of degree 2 (past the head-count
    bound): the second ring rank's query half visits its own key/value half
    (the causal diagonal) and the first half (every key), then merges the two
    partial results; also the fused form, where the first half's visit is merged
    into the running result in the same launch, and the gradients of both visits
    (ulysses_attention_chunk_backward, at 2.5x the forward flops).  Each call is
    timed in runs of its own; the figures are medians."""
    from sequence_long_context_amd import synth
    q, k, v = heads["q"][r], heads["k"][r], heads["v"][r]
    B, S, Hq, D = q.shape
    h = S // 2
    qb = q[:, h:].contiguous()
    kv = {"own": (k[:, h:].contiguous(), v[:, h:].contiguous(), h),
          "past": (k[:, :h].contiguous(), v[:, :h].contiguous(), 0)}
    o, lse = torch.empty_like(qb), torch.empty((B, Hq, S - h), dtype=torch.float32, device=dev)
    po, pl = torch.empty_like(o), torch.empty_like(lse)
    mo, ml = torch.empty_like(o), torch.empty_like(lse)
    # the fused form: the first half merged into a running result in the same launch
    ao, al = torch.empty_like(o), torch.empty_like(lse)
    U.ulysses_attention_chunk(qb, kv["own"][0], kv["own"][1], ao, al, causal, h, h)
    calls = {
        "chunk_own": lambda: U.ulysses_attention_chunk(qb, kv["own"][0], kv["own"][1], o, lse,
                                                       causal, h, h),
        "chunk_past": lambda: U.ulysses_attention_chunk(qb, kv["past"][0], kv["past"][1], po, pl,
                                                        causal, h, 0),
        # out of place, so that every timed call merges the same inputs
        "merge": lambda: U.ulysses_attention_merge(o, lse, po, pl, mo, ml),
        "chunk_past_accumulate": lambda: U.ulysses_attention_chunk_accumulate(
            qb, kv["past"][0], kv["past"][1], ao, al, causal, h, 0),
    }
    # gradients of the same visit pair: the output gradient of the query half,
    # the merged forward result (ao, al after the first fused call below), each
    # visit's dq added, dk and dv written per chunk
    g = torch.from_numpy(synth.normal(synth.seed_for(9, "do"), tuple(qb.shape)).view(np.int16))
    g = g.view(torch.bfloat16).to(dev)
    gq, gk, gv = torch.empty_like(qb), torch.empty_like(kv["own"][0]), torch.empty_like(kv["own"][0])
    delta = torch.empty_like(al)
    calls["chunk_backward_own"] = lambda: U.ulysses_attention_chunk_backward(
        qb, kv["own"][0], kv["own"][1], ao, g, al, delta, gq, gk, gv, causal, h, h)
    calls["chunk_backward_past"] = lambda: U.ulysses_attention_chunk_backward(
        qb, kv["past"][0], kv["past"][1], ao, g, al, delta, gq, gk, gv, causal, h, 0,
        accumulate_dq=True)
    # rounds of a few launches per call, the calls alternating in order from
    # round to round, medians over all launches; ~1 ms of queued work ahead of
    # each timed run, so that the stream never waits for the host between two
    # short launches
    samples = {name: [] for name in calls}
    for fn in calls.values():
        for _ in range(2):
            fn()
    torch.cuda.synchronize()
    for rnd in range(rounds):
        order = list(calls) if rnd % 2 == 0 else list(reversed(list(calls)))
        for name in order:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            calls["chunk_past"]()
            calls["chunk_past"]()
            ev[0].record()
            for i in range(reps):
                calls[name]()
                ev[i + 1].record()
            torch.cuda.synchronize()
            samples[name] += [ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(reps)]
    res = {name: float(np.median(v)) for name, v in samples.items()}
    rows = S - h
    f_own = attention_flops(rows, Hq, D, causal)
    f_past = 4.0 * D * B * Hq * rows * h
    mbytes = 3.0 * B * rows * Hq * D * 2 + 3.0 * B * Hq * rows * 4
    tot = res["chunk_own"] + res["chunk_past"] + res["merge"]
    return {
        "degree": 2, "query_rows": rows, "keys_per_visit": h,
        "chunk_own": {"TFLOP/s": round(f_own / res["chunk_own"] / 1e12, 2),
                      "us": round(res["chunk_own"] * 1e6, 2), "flops": f_own},
        "chunk_past": {"TFLOP/s": round(f_past / res["chunk_past"] / 1e12, 2),
                       "frac": round(f_past / res["chunk_past"] / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
                       "us": round(res["chunk_past"] * 1e6, 2), "flops": f_past},
        "merge": {"GB/s": round(mbytes / res["merge"] / 1e9, 1),
                  "frac_hbm": round(mbytes / res["merge"] / 1e9 / PEAK_HBM_GBPS, 4),
                  "us": round(res["merge"] * 1e6, 2), "bytes": mbytes},
        "rank_TFLOP/s": round((f_own + f_past) / tot / 1e12, 2),
        "chunk_past_accumulate": {
            "TFLOP/s": round(f_past / res["chunk_past_accumulate"] / 1e12, 2),
            "us": round(res["chunk_past_accumulate"] * 1e6, 2), "flops": f_past},
        "rank_TFLOP/s_fused": round((f_own + f_past) / (res["chunk_own"] + res["chunk_past_accumulate"])
                                    / 1e12, 2),
        "backward": {
            "own_us": round(res["chunk_backward_own"] * 1e6, 2),
            "past_us": round(res["chunk_backward_past"] * 1e6, 2),
            "TFLOP/s": round(2.5 * (f_own + f_past) / (res["chunk_backward_own"] + res["chunk_backward_past"])
                             / 1e12, 2),
            "flops": 2.5 * (f_own + f_past),
            "kernels": "attention_delta_kernel + attention_bwd_dq_kernel + attention_bwd_dkdv_kernel (chunk)"},
        "kernels": "attention_bf16_d128_kernel (chunk; accumulate) + merge_kernel",
    }


def time_split(U, torch, heads, r, causal, dev, rounds=6, reps=5):
    """The workload's sequence with one head per rank (P = the head count, the
    head-count bound): the plain attention call against ulysses_attention_local_split,
    whose key ranges of the long query blocks go to several workgroups and are merged
    in a second launch.  Calls alternate by round; medians.  Where the split's plan
    cuts nothing (the query blocks balance the GPU), only that is reported."""
    q, k, v = (heads[t][r][:, :, :1].contiguous() for t in "qkv")
    B, S, _, D = q.shape
    nbytes = U.ulysses_attention_local_split_workspace(B, S, 1, causal)
    if nbytes == 0:
        return {"heads": 1, "S": S, "split": False}
    ws = torch.empty((nbytes // 4,), dtype=torch.float32, device=dev)
    op, osp = torch.empty_like(q), torch.empty_like(q)
    calls = {"plain": lambda: U.ulysses_attention_local(q, k, v, op, causal),
             "split": lambda: U.ulysses_attention_local_split(q, k, v, osp, causal, ws)}
    samples = {name: [] for name in calls}
    for fn in calls.values():
        fn()
    torch.cuda.synchronize()
    for rnd in range(rounds):
        for name in (list(calls) if rnd % 2 == 0 else list(reversed(list(calls)))):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            ev[0].record()
            for i in range(reps):
                calls[name]()
                ev[i + 1].record()
            torch.cuda.synchronize()
            samples[name] += [ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(reps)]
    res = {name: float(np.median(v)) for name, v in samples.items()}
    f = attention_flops(S, 1, D, causal) * B
    return {"heads": 1, "S": S, "split": True, "workspace_bytes": nbytes,
            "plain": {"us": round(res["plain"] * 1e6, 2), "TFLOP/s": round(f / res["plain"] / 1e12, 2)},
            "split_call": {"us": round(res["split"] * 1e6, 2), "TFLOP/s": round(f / res["split"] / 1e12, 2)},
            "max_abs_diff_vs_plain": float((op.float() - osp.float()).abs().max().item()),
            "timing": f"median of {rounds} rounds x {reps} launches, call order alternating by round",
            "kernels": "attention_bf16_d128_kernel (split units) + split_merge_kernel"}


def time_pieces(U, torch, S, hq, hkv, D, P, causal, wid, dev, rounds=8, reps=5):
    """The rank's tokens as two batch entries (B = 2, S/2 tokens each), where the
    exchange's piece order [P][B][S/P][h][D] differs from [B][S][h][D]: the
    attention and its gradients reading and writing the piece order against the
    plain calls on unpacked copies, and the passes the piece order removes on a
    real rank (unpack of the received Q, K, V and pack of O into send order; in the
    backward, unpack of dO and pack of dQ, dK, dV), timed as device copies of
    permuted views, with their HBM-peak lower bound."""
    from sequence_long_context_amd import synth
    B, Sb = 2, S // 2
    Sp = Sb // P

    def up(seed, h):
        a = synth.normal(synth.seed_for(wid, seed), (P, B, Sp, h, D))
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    qp, kp, vp = up("pq", hq), up("pk", hkv), up("pv", hkv)
    op = torch.empty_like(qp)
    plain = [x.permute(1, 0, 2, 3, 4).reshape(B, Sb, -1, D).contiguous() for x in (qp, kp, vp)]
    ou = torch.empty_like(plain[0])

    def unpack_all():
        for src, dst in zip((qp, kp, vp), plain):
            dst.view(B, P, Sp, -1, D).copy_(src.permute(1, 0, 2, 3, 4))

    def pack_o():
        op.copy_(ou.view(B, P, Sp, hq, D).permute(1, 0, 2, 3, 4))

    # the gradients in the same two orders (output gradient: seeded, like the inputs)
    gp = up("do", hq)
    gu = gp.permute(1, 0, 2, 3, 4).reshape(B, Sb, hq, D).contiguous()
    lse = torch.empty((B, hq, Sb), dtype=torch.float32, device=dev)
    U.ulysses_attention_local_pieces(qp, kp, vp, op, causal, lse)
    U.ulysses_attention_local_lse(plain[0], plain[1], plain[2], ou, torch.empty_like(lse), causal)
    delta = torch.empty_like(lse)
    gpc = [torch.empty_like(x) for x in (qp, kp, vp)]
    gpl = [torch.empty_like(x) for x in plain]

    def unpack_do_pack_grads():
        gu.view(B, P, Sp, hq, D).copy_(gp.permute(1, 0, 2, 3, 4))
        for src, dst in zip(gpl, gpc):
            dst.copy_(src.view(B, P, Sp, -1, D).permute(1, 0, 2, 3, 4))

    calls = {
        "pieces": lambda: U.ulysses_attention_local_pieces(qp, kp, vp, op, causal),
        "plain": lambda: U.ulysses_attention_local(plain[0], plain[1], plain[2], ou, causal),
        "unpack_qkv": unpack_all,
        "pack_o": pack_o,
        "bwd_pieces": lambda: U.ulysses_attention_local_backward_pieces(qp, kp, vp, op, gp, lse, delta,
                                                                        *gpc, causal),
        "bwd_plain": lambda: U.ulysses_attention_local_backward(plain[0], plain[1], plain[2], ou, gu, lse,
                                                                delta, *gpl, causal),
        "bwd_passes": unpack_do_pack_grads,
    }
    # rounds of a few launches each, the calls alternating in order from round
    # to round, medians over all launches: the two attention forms are compared
    # under the same clock and cache history
    samples = {name: [] for name in calls}
    for fn in calls.values():
        for _ in range(2):
            fn()
    torch.cuda.synchronize()
    for rnd in range(rounds):
        order = list(calls) if rnd % 2 == 0 else list(reversed(list(calls)))
        for name in order:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            ev[0].record()
            for i in range(reps):
                calls[name]()
                ev[i + 1].record()
            torch.cuda.synchronize()
            samples[name] += [ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(reps)]
    res = {name: float(np.median(v)) for name, v in samples.items()}
    def packed(t):
        return t.view(B, P, Sp, -1, D).permute(1, 0, 2, 3, 4).contiguous().view(torch.int16)
    same = bool(torch.equal(op.view(torch.int16), packed(ou)))
    # both gradient calls ran last with the same inputs
    calls["bwd_plain"]()
    calls["bwd_pieces"]()
    torch.cuda.synchronize()
    same_bwd = all(bool(torch.equal(a.view(torch.int16), packed(b))) for a, b in zip(gpc, gpl))
    flops = attention_flops(Sb, hq, D, causal) * B
    removed_bytes = 2.0 * B * Sb * D * 2 * (2 * hq + 2 * hkv)  # read + write of Q, K, V and O
    return {
        "B": B, "S": Sb, "P": P, "piece_rows": Sp,
        "timing": f"median of {rounds} rounds x {reps} launches, call order alternating by round",
        "attention_pieces": {"us": round(res["pieces"] * 1e6, 2),
                             "TFLOP/s": round(flops / res["pieces"] / 1e12, 2)},
        "attention_plain": {"us": round(res["plain"] * 1e6, 2),
                            "TFLOP/s": round(flops / res["plain"] / 1e12, 2)},
        "bit_identical": same,
        "removed_passes": {"unpack_qkv_us": round(res["unpack_qkv"] * 1e6, 2),
                           "pack_o_us": round(res["pack_o"] * 1e6, 2),
                           "bytes": removed_bytes,
                           "us_at_hbm_peak": round(removed_bytes / (PEAK_HBM_GBPS * 1e9) * 1e6, 2),
                           "timed_as": "torch copy_ of a permuted view (what a rank would run)"},
        "backward": {"pieces_us": round(res["bwd_pieces"] * 1e6, 2),
                     "plain_us": round(res["bwd_plain"] * 1e6, 2),
                     "bit_identical": same_bwd,
                     "removed_passes_us": round(res["bwd_passes"] * 1e6, 2),
                     "removed_bytes": removed_bytes,
                     "removed_as": "unpack of dO and pack of dQ, dK, dV (torch copies of permuted views)"},
        "flops": flops,
        "kernels": "attention_bf16_d128_kernel (pieces) vs (plain); gradient kernels (pieces) vs (plain)",
    }


CPU_FLOPS_PER_THREAD = 2.5e9  # the oracle's fp64 rate per thread, for sizing the sample


def _rank_heads(a, B, S, P, h, r):
    """Rank r's heads [B][S][h][D] of a sequence-sharded tensor [P][B][S/P][H][D]."""
    D = a.shape[-1]
    g = a.transpose(1, 0, 2, 3, 4).reshape(B, S, h * P, D)
    return np.ascontiguousarray(g[:, :, r * h:(r + 1) * h, :])


def _oracle_attention_rate(q, k, v, causal, bf16, rows, threads):
    import oracle
    t0 = time.perf_counter()
    oracle.attention(q, k, v, causal, bf16=bf16, rows=rows, threads=threads)
    sec = time.perf_counter() - t0
    B, S, h, D = q.shape
    fl = attention_flops(S, h, D, causal, rows) * B
    return {"TFLOP/s": fl / sec / 1e12, "sec": round(sec, 3), "flops": fl, "threads": threads,
            "rows": S if rows is None else int(np.asarray(rows).size)}


def cpu_baseline(host, B, S, Hq, Hkv, D, P, hq, hkv, r, dt, causal, stride, wname, wid):
    """The fp64 CPU oracle (as it stands) on the host cores:
    value        rank r's attention over the timed workload, every query row when that
                 is estimated under ~30 s on these cores (else every stride-th row);
    transposes   the oracle's seq->head of Q, K, V and head->seq of O, all P shards, in
                 full (single-threaded byte copies);
    small        the full attention of the two small workloads (tiny fp32, s4k bf16) on
                 all threads and on one core, and their layout changes in full."""
    import oracle
    from sequence_long_context_amd import synth

    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    threads = max(1, min(threads, os.cpu_count() or 1))
    q, k, v = (_rank_heads(host[t], B, S, P, h, r) for t, h in (("q", hq), ("k", hkv), ("v", hkv)))
    if stride <= 0:
        stride = 1
        full = attention_flops(S, hq, D, causal) * B
        while full / stride / (CPU_FLOPS_PER_THREAD * threads) > 30.0:
            stride *= 2
    rows = None if stride == 1 else np.arange(0, S, stride, dtype=np.int64)
    main = _oracle_attention_rate(q, k, v, causal, dt == "bf16", rows, threads)

    # the layout changes of the whole step, in full
    lay = {}
    for name, a in (("q_s2h", host["q"]), ("k_s2h", host["k"]), ("v_s2h", host["v"])):
        t0 = time.perf_counter()
        oracle.seq_to_head(a, P)
        lay[name] = time.perf_counter() - t0
    o_head = oracle.seq_to_head(host["q"], P)  # an output-shaped head-layout buffer
    t0 = time.perf_counter()
    oracle.head_to_seq(o_head, P)
    lay["o_h2s"] = time.perf_counter() - t0
    del o_head
    lay_bytes = 2.0 * sum(host[t].nbytes for t in ("q", "k", "v", "q"))  # read + write
    lay_sec = sum(lay.values())

    small = {}
    for name in ("tiny", "s4k"):
        swid, sB, sS, sHq, sHkv, sD, sP, sdt, scausal = WORKLOADS[name]
        sq, sk, sv = (synth.normal(synth.seed_for(swid, t), (sP, sB, sS // sP, H, sD), sdt)
                      for t, H in (("q", sHq), ("k", sHkv), ("v", sHkv)))
        args_ = [_rank_heads(a, sB, sS, sP, H // sP, 0) for a, H in ((sq, sHq), (sk, sHkv), (sv, sHkv))]
        o_head = oracle.seq_to_head(sq, sP)  # an output-shaped head-layout buffer
        t0 = time.perf_counter()
        for a in (sq, sk, sv):
            oracle.seq_to_head(a, sP)
        oracle.head_to_seq(o_head, sP)
        tsec = time.perf_counter() - t0
        tbytes = 2.0 * (sq.nbytes * 2 + sk.nbytes + sv.nbytes)  # Q, K, V seq->head, O head->seq
        small[name] = {
            "all_threads": _oracle_attention_rate(*args_, scausal, sdt == "bf16", None, threads),
            "one_core": _oracle_attention_rate(*args_, scausal, sdt == "bf16", None, 1),
            "transposes": {"GB/s": round(tbytes / tsec / 1e9, 4), "sec": round(tsec, 4), "cores": 1,
                           "bytes": tbytes, "note": "Q, K, V seq->head and O head->seq in full"},
        }
        for key in ("all_threads", "one_core"):
            small[name][key]["TFLOP/s"] = round(small[name][key]["TFLOP/s"], 6)

    sample = (f"{wname} rank {r}: " + ("every query row" if stride == 1 else f"every {stride}th query row")
              + f" ({main['rows']} rows x {hq} heads, {main['flops']:.3e} flop) in {main['sec']:.2f} s "
              f"on {threads} threads, fp64 two-pass softmax")
    return {"value": main["TFLOP/s"], "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample,
            "transposes": {"GB/s": round(lay_bytes / lay_sec / 1e9, 4), "sec": round(lay_sec, 3),
                           "bytes": lay_bytes, "cores": 1,
                           "per_call_sec": {k_: round(v_, 3) for k_, v_ in lay.items()},
                           "sample": f"{wname}: seq->head of Q, K, V and head->seq of O, all {P} "
                                     f"shards, in full (byte copies, one thread)"},
            "small": small}


if __name__ == "__main__":
    main()
