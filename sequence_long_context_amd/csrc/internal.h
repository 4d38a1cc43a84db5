// Internal declarations shared by the translation units of libulysses.so.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace uly {

// Unsigned 32-bit division by a run-time constant as multiply-high + shift
// (Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication", 1994, round-up method).  Exact for every n < 2^32.
struct FastDiv {
    uint32_t d, m, s;
    FastDiv() : d(1), m(1), s(0) {}
    explicit FastDiv(uint32_t div) : d(div) {
        s = 0;
        while ((uint64_t(1) << s) < div) ++s;
        m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << s) - div)) / div + 1);
    }
    __host__ __device__ inline uint32_t div(uint32_t n) const {
        uint64_t t = (uint64_t(n) * m) >> 32;
        return uint32_t((t + n) >> s);
    }
};

// Layout change between SEQ[P][B][S/P][H][D] and HEAD[P][B][S][H/P][D], or
// with pieces PIECES[P][P][B][S/P][H/P][D] (the pieces of each rank in
// source-rank order), element size `elem` bytes.  Arguments are validated by
// the caller.
hipError_t launch_layout(const void *src, void *dst, int64_t B, int64_t S, int64_t H,
                         int64_t D, int32_t P, int32_t elem, bool to_head, bool pieces,
                         hipStream_t st);

// seq->head (or seq->pieces) of Q (Hq heads), K and V (Hkv heads) in one launch.
hipError_t launch_layout_qkv(const void *const src[3], void *const dst[3], int64_t B, int64_t S,
                             int64_t Hq, int64_t Hkv, int64_t D, int32_t P, int32_t elem,
                             bool pieces, hipStream_t st);

// bf16 attention, head_dim 128, MFMA kernel; lse ([B][Hq][S], natural log of
// each row's sum of exp(scores)) is written when not NULL.  sp = 0: q, k, v,
// o are [B][S][h][D]; sp > 0: they are in pieces [S/sp][B][sp][h][D] (sp a
// multiple of 64 when B > 1).
hipError_t launch_attention_bf16_d128(const void *q, const void *k, const void *v, void *o,
                                      float *lse, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                      int64_t sp, bool causal, hipStream_t st);

// Split gradients (bf16, head_dim 128, full sequence in [B][S][h][D]): the
// gradients of ulysses_attention_local_backward with the longest dK/dV key
// blocks' query streams cut into units on several workgroups, fp32 partial
// sums in the workspace, added in unit order by a second launch.
// Workspace bytes for these sizes (0: nothing is split, and the launch is the
// plain call's).
uint64_t attention_bwd_bf16_d128_split_workspace(int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                                 bool causal);
hipError_t launch_attention_bwd_bf16_d128_split(const void *q, const void *k, const void *v,
                                                const void *o, const void *dout, const float *lse,
                                                float *delta, void *dq, void *dk, void *dv, int64_t B,
                                                int64_t S, int64_t Hq, int64_t Hkv, bool causal,
                                                void *workspace, hipStream_t st);

// Split forward (bf16, head_dim 128, full sequence in [B][S][h][D]): each
// 64-row query block's key tiles cut into units handled by different
// workgroups, fp32 partial results in the workspace, merged by their share of
// the exp-sum in a second launch.  Workspace bytes for these sizes (0: nothing
// is split, and the launch is the plain call's).  lse may be NULL.
uint64_t attention_bf16_d128_split_workspace(int64_t B, int64_t S, int64_t Hq, bool causal);
hipError_t launch_attention_bf16_d128_split(const void *q, const void *k, const void *v, void *o,
                                            float *lse, int64_t B, int64_t S, int64_t Hq,
                                            int64_t Hkv, bool causal, void *workspace,
                                            hipStream_t st);

// fp32 attention, head_dim 32/64/128, vector-ALU kernel; lse and sp as above
// (any sp dividing S).
hipError_t launch_attention_f32(const float *q, const float *k, const float *v, float *o,
                                float *lse, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                int64_t D, int64_t sp, bool causal, hipStream_t st);

// Attention of Sq query rows over one chunk of Skv keys (key j visible to
// row i under the causal mask iff j <= i + delta); rows with no visible key
// get o = 0 and lse = -inf.  bf16 with head_dim 128, and fp32.  With
// accumulate (bf16), o and lse hold a running result that this chunk is
// merged into; rows the chunk does not reach are left as they are.
hipError_t launch_attention_chunk_bf16_d128(const void *q, const void *k, const void *v, void *o,
                                            float *lse, int64_t B, int64_t Sq, int64_t Skv,
                                            int64_t delta, int64_t Hq, int64_t Hkv, bool causal,
                                            bool accumulate, hipStream_t st);
hipError_t launch_attention_chunk_f32(const float *q, const float *k, const float *v, float *o,
                                      float *lse, int64_t B, int64_t Sq, int64_t Skv,
                                      int64_t delta, int64_t Hq, int64_t Hkv, int64_t D,
                                      bool causal, hipStream_t st);

// Merge of two partial results (o [B][S][H][D], lse [B][H][S]); head_dim *
// elem is a power of two in [16, 1024].
hipError_t launch_merge(const void *oa, const float *lse_a, const void *ob, const float *lse_b,
                        void *o, float *lse, int64_t B, int64_t S, int64_t H, int64_t D, int32_t elem,
                        hipStream_t st);

// Gradients of the bf16 attention (head_dim 128): delta ([B][Hq][S]) is
// scratch supplied by the caller; sp as for the forward (0: [B][S][h][D]).
hipError_t launch_attention_bwd_bf16_d128(const void *q, const void *k, const void *v,
                                          const void *o, const void *dout, const float *lse,
                                          float *delta, void *dq, void *dk, void *dv, int64_t B,
                                          int64_t S, int64_t Hq, int64_t Hkv, int64_t sp,
                                          bool causal, hipStream_t st);

// Gradient contributions of one key/value chunk (Sq query rows, Skv keys, key
// j visible to row i under the causal mask iff j <= i + dpos), from the
// merged output and log-sum-exp; with acc_dq / acc_dkv they are added to dq /
// to dk and dv.
hipError_t launch_attention_chunk_bwd_bf16_d128(const void *q, const void *k, const void *v,
                                                const void *o, const void *dout, const float *lse,
                                                float *delta, void *dq, void *dk, void *dv,
                                                int64_t B, int64_t Sq, int64_t Skv, int64_t dpos,
                                                bool acc_dq, bool acc_dkv, int64_t Hq, int64_t Hkv,
                                                bool causal, hipStream_t st);

// Capacity (in floats) of each GPU's file-scope scratch array, and its device
// address on the device of `stream` (NULL: the current device), looked up once
// per device.
constexpr int64_t kScratchFloats = int64_t(1) << 20;  // 4 MiB per GPU
hipError_t scratch_floats(void *stream, float **ptr);

}  // namespace uly
