// The chain-split instantiations of the bf16 attention kernel (64-row blocks,
// key split and chain split; the kernel and its design notes are in
// attn_fwd.h and attention_bf16.hip), plain and as split-forward units.
//
// They live in a source file of their own so that they can be built with
// the instruction scheduler's "max-memory-clause" strategy (the build passes
// -mllvm -amdgpu-sched-strategy=max-memory-clause for this file only).
// Measured on MI355X, alternating libraries, same outputs: S = 4096 with 4
// heads, causal, 44.6 -> 43.8 us; S = 8192 95.9 -> 94.2 us; the split forward
// with one head, S = 4096 32.5 -> 30.9 us, S = 8192 45.2 -> 44.1 us.  The same
// strategy made the 256-row blocks slower (32768 tokens, causal: 940.4 ->
// 955.9 us), so attention_bf16.hip keeps the default.
#include "attn_fwd.h"

namespace uly {

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
