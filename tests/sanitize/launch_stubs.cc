// Host-only stand-ins for the kernel launchers of libulysses.so, so that the
// C-ABI's argument checks and dispatch (csrc/api.hip) can be built and run
// under AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a
// GPU.  Each stand-in records that it was reached and the sizes it was given;
// nothing is launched and no device memory is touched.
#include "../../sequence_long_context_amd/csrc/internal.h"

#include "stub_record.h"

StubRecord g_stub;

namespace {
hipError_t reached(const char *what, int64_t a, int64_t b, int64_t c, int64_t d) {
    ++g_stub.calls;
    g_stub.last = what;
    g_stub.sizes[0] = a;
    g_stub.sizes[1] = b;
    g_stub.sizes[2] = c;
    g_stub.sizes[3] = d;
    return hipSuccess;
}
}  // namespace

extern "C" const char *hipGetErrorString(hipError_t) { return "stub error string"; }

namespace uly {
hipError_t launch_layout(const void *, void *, int64_t B, int64_t S, int64_t H, int64_t D, int32_t,
                         int32_t, bool, bool pieces, hipStream_t) {
    g_stub.layout = pieces;
    return reached("layout", B, S, H, D);
}
hipError_t launch_layout_qkv(const void *const[3], void *const[3], int64_t B, int64_t S, int64_t Hq,
                             int64_t Hkv, int64_t, int32_t, int32_t, bool pieces, hipStream_t) {
    g_stub.layout = pieces;
    return reached("layout_qkv", B, S, Hq, Hkv);
}
hipError_t launch_attention_bf16_d128(const void *, const void *, const void *, void *, float *,
                                      int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t sp,
                                      bool, hipStream_t) {
    g_stub.layout = sp;
    return reached("attention_bf16", B, S, Hq, Hkv);
}
uint64_t attention_bf16_d128_split_workspace(int64_t B, int64_t S, int64_t Hq, bool) {
    return S <= 8192 ? uint64_t(B * Hq) * 4096u : 0;  // some short sizes need a workspace
}
hipError_t launch_attention_bf16_d128_split(const void *, const void *, const void *, void *,
                                            float *, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                            bool, void *, hipStream_t) {
    return reached("split", B, S, Hq, Hkv);
}
hipError_t launch_attention_f32(const float *, const float *, const float *, float *, float *,
                                int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t, int64_t sp,
                                bool, hipStream_t) {
    g_stub.layout = sp;
    return reached("attention_f32", B, S, Hq, Hkv);
}
hipError_t launch_attention_chunk_bf16_d128(const void *, const void *, const void *, void *,
                                            float *, int64_t B, int64_t Sq, int64_t Skv,
                                            int64_t delta, int64_t, int64_t, bool, bool,
                                            hipStream_t) {
    return reached("chunk_bf16", B, Sq, Skv, delta);
}
hipError_t launch_attention_chunk_f32(const float *, const float *, const float *, float *, float *,
                                      int64_t B, int64_t Sq, int64_t Skv, int64_t delta, int64_t,
                                      int64_t, int64_t, bool, hipStream_t) {
    return reached("chunk_f32", B, Sq, Skv, delta);
}
hipError_t launch_merge(const void *, const float *, const void *, const float *, void *, float *,
                        int64_t B, int64_t S, int64_t H, int64_t D, int32_t, hipStream_t) {
    return reached("merge", B, S, H, D);
}
hipError_t launch_attention_bwd_bf16_d128(const void *, const void *, const void *, const void *,
                                          const void *, const float *, float *, void *, void *,
                                          void *, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                          int64_t sp, bool, hipStream_t) {
    g_stub.layout = sp;
    return reached("backward", B, S, Hq, Hkv);
}
hipError_t scratch_floats(void *, float **ptr) {
    *ptr = reinterpret_cast<float *>(uintptr_t(0x7FF000000000));  // never dereferenced
    return hipSuccess;
}
hipError_t launch_attention_chunk_bwd_bf16_d128(const void *, const void *, const void *,
                                                const void *, const void *, const float *, float *,
                                                void *, void *, void *, int64_t B, int64_t Sq,
                                                int64_t Skv, int64_t dpos, bool, bool, int64_t,
                                                int64_t, bool, hipStream_t) {
    return reached("chunk_backward", B, Sq, Skv, dpos);
}
uint64_t attention_bwd_bf16_d128_split_workspace(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, bool) {
    return uint64_t(B) * uint64_t(S) * uint64_t(Hq + Hkv) % 3 ? 1u << 20 : 0u;  // some sizes need one
}
hipError_t launch_attention_bwd_bf16_d128_split(const void *, const void *, const void *, const void *,
                                                const void *, const float *, float *, void *, void *,
                                                void *, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                                bool, void *, hipStream_t) {
    return reached("backward_split", B, S, Hq, Hkv);
}
}  // namespace uly
