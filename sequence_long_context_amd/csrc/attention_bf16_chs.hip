// The chain-split instantiations of the bf16 attention kernel (64-row blocks,
// key split and chain split; the kernel and its design notes are in
// attn_fwd.h and attention_bf16.hip), plain and as split-forward units, and
// the merge of the split forward's units.
//
// They live in a source file of their own so that they can be built with
// the instruction scheduler's "max-memory-clause" strategy (the build passes
// -mllvm -amdgpu-sched-strategy=max-memory-clause for this file only).
// Measured on MI355X, alternating libraries, same outputs: S = 4096 with 4
// heads, causal, 44.6 -> 43.8 us; S = 8192 95.9 -> 94.2 us; the split forward
// with one head, S = 4096 32.5 -> 30.9 us, S = 8192 45.2 -> 44.1 us.  The same
// strategy made the 256-row blocks slower (32768 tokens, causal: 940.4 ->
// 955.9 us), so attention_bf16.hip keeps the default.  The merge kernel is
// here for the same reason: with it in this file the split calls took 33.2 ->
// 31.4 us (S = 4096, one head), 46.1 -> 45.2 (8192), 34.0 -> 33.2 (4096, two
// heads).
#include "attn_fwd.h"

namespace uly {
namespace {
// Merge of a split block's units: per row, with lse_u and o_u the units'
// log-sum-exp and normalised fp32 output (attention over disjoint key ranges),
//   lse = log sum_u exp(lse_u),   o = sum_u exp(lse_u - lse) o_u,
// taken against the largest lse_u and rounded to bf16 once.  One workgroup per
// (split query block, head); four threads per row, 32 columns each.
__global__ __launch_bounds__(256) void split_merge_kernel(const float *__restrict__ ws,
                                                          short *__restrict__ o,
                                                          float *__restrict__ lse, int S, int Hq,
                                                          int nqb, int umax, int ctiles, int first,
                                                          int causal) {
    const int qb = first + int(blockIdx.x), hh = int(blockIdx.y);
    const int nunits = ((causal ? qb + 1 : nqb) + ctiles - 1) / ctiles;
    const int r = int(threadIdx.x) >> 2, d0 = (int(threadIdx.x) & 3) * 32;
    const int qrow = qb * kSplitRows + r;
    if (qrow >= S) return;
    const float *slot = ws + (int64_t(hh) * nqb + qb) * umax * kSplitSlot;
    const float *ls = slot + kSplitRows * kD + r;
    float m = -INFINITY;
    for (int u = 0; u < nunits; ++u) m = fmaxf(m, ls[u * kSplitSlot]);
    float tot = 0.f;
    for (int u = 0; u < nunits; ++u) tot += expf(ls[u * kSplitSlot] - m);
    const float L = m == -INFINITY ? -INFINITY : m + logf(tot);
    f32x4 acc[8] = {};
    if (m != -INFINITY)
        for (int u = 0; u < nunits; ++u) {
            const float wgt = expf(ls[u * kSplitSlot] - L);
            const f32x4 *src = reinterpret_cast<const f32x4 *>(slot + u * kSplitSlot + r * kD + d0);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += wgt * src[i];
        }
    const int b = hh / Hq, head = hh - b * Hq;
    short *dst = o + ((int64_t(b) * S + qrow) * Hq + head) * kD + d0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s16x8 pv;
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = to_bf16(acc[2 * i + j / 4][j % 4]);
        *reinterpret_cast<s16x8 *>(dst + 8 * i) = pv;
    }
    if (lse && (threadIdx.x & 3) == 0) lse[int64_t(hh) * S + qrow] = L;
}

}  // namespace

hipError_t launch_split_merge(const float *ws, void *o, float *lse, int S, int Hq, int nqb, int umax,
                              int ctiles, int first, int htot, bool causal, hipStream_t st) {
    hipLaunchKernelGGL(split_merge_kernel, dim3(uint32_t(nqb - first), uint32_t(htot)), dim3(256), 0, st,
                       ws, static_cast<short *>(o), lse, S, Hq, nqb, umax, ctiles, first, causal ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_chain_split(const void *q, const void *k, const void *v, void *o, float *lse,
                              int64_t B, int64_t Sq, int64_t Skv, int64_t delta, int64_t Hq,
                              int64_t Hkv, bool causal, bool chunk, bool acc, int64_t sp, int cus,
                              hipStream_t st) {
    return launch_nw<8, 2, true>(q, k, v, o, lse, B, Sq, Skv, delta, Hq, Hkv, causal, chunk, acc, sp, cus, st);
}

hipError_t launch_split_units(dim3 grid, hipStream_t st, const void *q, const void *k, const void *v,
                              void *o, float *lse, int S, int Hq, int Hkv, int nqb, int htot,
                              bool causal, const SplitTable &t) {
    const float scale_log2 = float(1.4426950408889634 / 11.313708498984761);  // log2(e)/sqrt(128)
    if (causal)
        launch_one<true, 8, false, 2, false, false, true, true>(grid, st, q, k, v, o, lse, S, S, 0, Hq, Hkv,
                                                                nqb, htot, 0, scale_log2, FastDiv(), 0, t);
    else
        launch_one<false, 8, false, 2, false, false, true, true>(grid, st, q, k, v, o, lse, S, S, 0, Hq, Hkv,
                                                                 nqb, htot, 0, scale_log2, FastDiv(), 0, t);
    return hipGetLastError();
}

}  // namespace uly
