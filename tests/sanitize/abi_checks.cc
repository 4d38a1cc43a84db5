// Argument checks of the C ABI (include/ulysses.h) run on the host, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (no recovery) together with
// csrc/api.hip and the stand-in launchers of launch_stubs.cc.  Every entry
// point is called with accepted arguments (the stand-in must be reached with
// the caller's sizes) and with each kind of rejected argument, including sizes
// whose products overflow 64 bits, which must be refused without undefined
// behaviour.  Exit status 0: every expectation held and no sanitizer report.
#include "../../include/ulysses.h"
#include "stub_record.h"

#include <cstdint>
#include <cstdio>
#include <cstring>

namespace {
int failures = 0;
// dummy device addresses: never dereferenced (the launches are stand-ins)
char *const A = reinterpret_cast<char *>(uintptr_t(0x7F0000000000));
char *const B_ = reinterpret_cast<char *>(uintptr_t(0x7F1000000000));
char *const C = reinterpret_cast<char *>(uintptr_t(0x7F2000000000));
char *const D_ = reinterpret_cast<char *>(uintptr_t(0x7F3000000000));
char *const E = reinterpret_cast<char *>(uintptr_t(0x7F4000000000));
char *const F = reinterpret_cast<char *>(uintptr_t(0x7F5000000000));
char *const G = reinterpret_cast<char *>(uintptr_t(0x7F6000000000));
char *const H = reinterpret_cast<char *>(uintptr_t(0x7F7000000000));
char *const I = reinterpret_cast<char *>(uintptr_t(0x7F8000000000));
char *const J = reinterpret_cast<char *>(uintptr_t(0x7F9000000000));
float *fl(char *p) { return reinterpret_cast<float *>(p); }
const int64_t kHuge = int64_t(1) << 40, kBig = int64_t(1) << 62, kMax = INT64_MAX;

void expect(bool ok, const char *what, int line) {
    if (!ok) {
        ++failures;
        std::fprintf(stderr, "line %d: %s (last error: %s)\n", line, what, ulysses_last_error());
    }
}
#define EXPECT_STATUS(call, st) expect((call) == (st), #call " == " #st, __LINE__)
#define EXPECT_LAUNCH(call, name, a, b)                                                        \
    do {                                                                                       \
        const int before = g_stub.calls;                                                       \
        expect((call) == ULY_OK, #call " == ULY_OK", __LINE__);                                \
        expect(g_stub.calls == before + 1 && std::strcmp(g_stub.last, name) == 0 &&            \
                   g_stub.sizes[0] == (a) && g_stub.sizes[1] == (b),                           \
               #call " reaches " name, __LINE__);                                              \
    } while (0)
#define EXPECT_NO_LAUNCH(call, st)                                                             \
    do {                                                                                       \
        const int before = g_stub.calls;                                                       \
        expect((call) == (st), #call " == " #st, __LINE__);                                    \
        expect(g_stub.calls == before, #call " launches nothing", __LINE__);                   \
    } while (0)
}  // namespace

int main() {
    const uly_dtype_t bf = ULY_DTYPE_BF16, f32 = ULY_DTYPE_FP32;
    // layout changes
    for (int dir = 0; dir < 2; ++dir) {
        auto lay = [&](const void *s, void *d, int64_t B, int64_t S, int64_t Hh, int64_t Dd,
                       int32_t P, uly_dtype_t dt) {
            return dir ? ulysses_head_to_seq(s, d, B, S, Hh, Dd, P, dt, nullptr)
                       : ulysses_seq_to_head(s, d, B, S, Hh, Dd, P, dt, nullptr);
        };
        EXPECT_LAUNCH(lay(A, B_, 2, 64, 8, 128, 4, bf), "layout", 2, 64);
        EXPECT_NO_LAUNCH(lay(A, B_, 0, 64, 8, 128, 4, bf), ULY_OK);  // empty
        EXPECT_NO_LAUNCH(lay(nullptr, B_, 1, 64, 8, 128, 4, bf), ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(lay(A + 1, B_, 1, 64, 8, 128, 4, bf), ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(lay(A, A + 64, 1, 64, 8, 128, 4, bf), ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(lay(A, B_, 1, 63, 8, 128, 4, bf), ULY_ERR_NOT_DIVISIBLE);
        EXPECT_NO_LAUNCH(lay(A, B_, 1, 64, 4, 128, 8, bf), ULY_ERR_NOT_DIVISIBLE);
        EXPECT_NO_LAUNCH(lay(A, B_, -1, 64, 8, 128, 4, bf), ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(lay(A, B_, 1, 64, 8, 128, 4, uly_dtype_t(7)), ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(lay(A, B_, kHuge, kHuge, 8, 128, 4, bf), ULY_ERR_UNSUPPORTED);
        EXPECT_NO_LAUNCH(lay(A, B_, kBig, kBig, kBig, kBig, 4, bf), ULY_ERR_UNSUPPORTED);
        EXPECT_NO_LAUNCH(lay(A, B_, kMax, kMax, kMax, kMax, 4, bf), ULY_ERR_NOT_DIVISIBLE);
        EXPECT_NO_LAUNCH(lay(A, B_, 1, 1 << 30, 1 << 30, 16, 1 << 30, f32), ULY_ERR_UNSUPPORTED);
    }
    EXPECT_LAUNCH(ulysses_seq_to_head_qkv(A, B_, C, D_, E, F, 1, 64, 8, 4, 128, 4, bf, nullptr),
                  "layout_qkv", 1, 64);
    EXPECT_NO_LAUNCH(ulysses_seq_to_head_qkv(A, B_, C, D_, D_, F, 1, 64, 8, 4, 128, 4, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_seq_to_head_qkv(A, B_, C, D_, E, F, kBig, kBig, kBig, kBig, kBig, 4, bf,
                                             nullptr),
                     ULY_ERR_UNSUPPORTED);

    // the exchanges with their pieces left as delivered
    EXPECT_LAUNCH(ulysses_seq_to_pieces(A, B_, 2, 64, 8, 128, 4, bf, nullptr), "layout", 2, 64);
    expect(g_stub.layout == 1, "seq_to_pieces launches the pieces layout", __LINE__);
    EXPECT_LAUNCH(ulysses_seq_to_head(A, B_, 2, 64, 8, 128, 4, bf, nullptr), "layout", 2, 64);
    expect(g_stub.layout == 0, "seq_to_head launches the head layout", __LINE__);
    EXPECT_LAUNCH(ulysses_pieces_to_seq(A, B_, 2, 64, 8, 128, 4, bf, nullptr), "layout", 2, 64);
    expect(g_stub.layout == 1, "pieces_to_seq launches the pieces layout", __LINE__);
    EXPECT_LAUNCH(ulysses_seq_to_pieces_qkv(A, B_, C, D_, E, F, 3, 64, 8, 4, 128, 4, bf, nullptr),
                  "layout_qkv", 3, 64);
    expect(g_stub.layout == 1, "seq_to_pieces_qkv launches the pieces layout", __LINE__);
    EXPECT_NO_LAUNCH(ulysses_seq_to_pieces(A, B_, 1, 63, 8, 128, 4, bf, nullptr), ULY_ERR_NOT_DIVISIBLE);
    EXPECT_NO_LAUNCH(ulysses_pieces_to_seq(A, A + 2, 1, 64, 8, 128, 4, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_seq_to_pieces_qkv(A, B_, C, D_, E, E, 1, 64, 8, 4, 128, 4, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_seq_to_pieces(A, B_, kMax, kMax, kMax, kMax, 4, bf, nullptr),
                     ULY_ERR_NOT_DIVISIBLE);
    EXPECT_LAUNCH(ulysses_attention_local_pieces(A, B_, C, D_, nullptr, 2, 512, 4, 2, 128, 8, 1, bf,
                                                 nullptr),
                  "attention_bf16", 2, 512);
    expect(g_stub.layout == 64, "attention_local_pieces passes rows per piece", __LINE__);
    EXPECT_LAUNCH(ulysses_attention_local_pieces(A, B_, C, D_, fl(E), 3, 96, 4, 4, 64, 8, 0, f32,
                                                 nullptr),
                  "attention_f32", 3, 96);
    expect(g_stub.layout == 12, "fp32 pieces of any height", __LINE__);
    EXPECT_LAUNCH(ulysses_attention_local_pieces(A, B_, C, D_, nullptr, 1, 100, 4, 2, 128, 4, 1, bf,
                                                 nullptr),
                  "attention_bf16", 1, 100);  // one batch entry: pieces of any height
    EXPECT_NO_LAUNCH(ulysses_attention_local_pieces(A, B_, C, D_, nullptr, 2, 96, 4, 2, 128, 3, 1, bf,
                                                    nullptr),
                     ULY_ERR_UNSUPPORTED);  // 32-row pieces with two batch entries
    EXPECT_NO_LAUNCH(ulysses_attention_local_pieces(A, B_, C, D_, nullptr, 2, 100, 4, 2, 128, 3, 1,
                                                    bf, nullptr),
                     ULY_ERR_NOT_DIVISIBLE);
    EXPECT_NO_LAUNCH(ulysses_attention_local_pieces(A, B_, C, D_, nullptr, 2, 128, 4, 2, 128, 0, 1,
                                                    bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_attention_local_pieces(A, B_, C, D_, nullptr, kMax, kMax, kMax, 1, 128,
                                                    2, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(ulysses_attention_local_pieces(A, B_, C, D_, nullptr, 0, 128, 4, 2, 128, 2, 1, bf,
                                                    nullptr),
                     ULY_OK);

    // attention forward
    EXPECT_LAUNCH(ulysses_attention_local(A, B_, C, D_, 2, 100, 4, 2, 128, 1, bf, nullptr),
                  "attention_bf16", 2, 100);
    expect(g_stub.layout == 0, "attention_local reads [B][S][h][D]", __LINE__);
    EXPECT_LAUNCH(ulysses_attention_local(A, B_, C, D_, 1, 100, 4, 2, 64, 0, f32, nullptr),
                  "attention_f32", 1, 100);
    EXPECT_LAUNCH(ulysses_attention_local_lse(A, B_, C, D_, fl(E), 1, 100, 4, 2, 128, 1, bf, nullptr),
                  "attention_bf16", 1, 100);
    EXPECT_NO_LAUNCH(ulysses_attention_local(A, B_, C, D_, 0, 100, 4, 2, 128, 1, bf, nullptr), ULY_OK);
    EXPECT_NO_LAUNCH(ulysses_attention_local(A, B_, C, D_, 1, 100, 4, 3, 128, 1, bf, nullptr),
                     ULY_ERR_NOT_DIVISIBLE);
    EXPECT_NO_LAUNCH(ulysses_attention_local(A, B_, C, D_, 1, 100, 4, 2, 96, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(ulysses_attention_local(A, B_, C, A, 1, 100, 4, 2, 128, 1, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_attention_local(A + 8, B_, C, D_, 1, 100, 4, 2, 128, 1, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_attention_local_lse(A, B_, C, D_, nullptr, 1, 100, 4, 2, 128, 1, bf,
                                                 nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    // products of B, S and the head counts beyond 64 bits are refused, not wrapped
    EXPECT_NO_LAUNCH(ulysses_attention_local(A, B_, C, D_, int64_t(1) << 32, 64, int64_t(1) << 32, 1,
                                             128, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(ulysses_attention_local(A, B_, C, D_, kMax, 1, kMax, kMax, 128, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(ulysses_attention_local(A, B_, C, D_, 1, kMax, 1, 1, 128, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);

    // split forward: workspace query and the call
    {
        uint64_t n = 7;
        EXPECT_STATUS(ulysses_attention_local_split_workspace(2, 4096, 4, 128, 1, bf, &n), ULY_OK);
        expect(n == 2 * 4 * 4096, "split workspace reported", __LINE__);
        EXPECT_STATUS(ulysses_attention_local_split_workspace(1, 65536, 4, 128, 1, bf, &n), ULY_OK);
        expect(n == 0, "no split workspace for long sequences", __LINE__);
        EXPECT_STATUS(ulysses_attention_local_split_workspace(1, 4096, 4, 128, 1, bf, nullptr),
                      ULY_ERR_INVALID_ARGUMENT);
        EXPECT_STATUS(ulysses_attention_local_split_workspace(1, 4096, 4, 64, 1, f32, &n),
                      ULY_ERR_UNSUPPORTED);
        EXPECT_STATUS(ulysses_attention_local_split_workspace(1, 4096, 65536, 128, 1, bf, &n),
                      ULY_ERR_UNSUPPORTED);
        EXPECT_STATUS(ulysses_attention_local_split_workspace(kMax, kMax, 4, 128, 1, bf, &n),
                      ULY_ERR_UNSUPPORTED);
        const uint64_t need = 4 * 4096;
        EXPECT_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, fl(E), 1, 4096, 4, 2, 128, 1, bf, F,
                                                    need, nullptr),
                      "split", 1, 4096);
        EXPECT_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, nullptr, 1, 65536, 4, 2, 128, 1, bf,
                                                    nullptr, 0, nullptr),
                      "split", 1, 65536);
        EXPECT_NO_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, nullptr, 1, 4096, 4, 2, 128, 1, bf,
                                                       F, need - 16, nullptr),
                         ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, nullptr, 1, 4096, 4, 2, 128, 1, bf,
                                                       nullptr, need, nullptr),
                         ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, nullptr, 1, 4096, 4, 2, 128, 1, bf,
                                                       F + 8, need, nullptr),
                         ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, nullptr, 1, 4096, 4, 2, 128, 1, bf,
                                                       A + 64, need, nullptr),
                         ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, fl(E), 1, 4096, 4, 2, 128, 1, bf,
                                                       E + 4096, need, nullptr),
                         ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(ulysses_attention_local_split(A, B_, C, A, nullptr, 1, 4096, 4, 2, 128, 1, bf,
                                                       F, need, nullptr),
                         ULY_ERR_INVALID_ARGUMENT);
        EXPECT_NO_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, nullptr, 1, 4096, 4, 2, 64, 1, f32,
                                                       F, need, nullptr),
                         ULY_ERR_UNSUPPORTED);
        EXPECT_NO_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, nullptr, 0, 4096, 4, 2, 128, 1, bf,
                                                       nullptr, 0, nullptr),
                         ULY_OK);
        EXPECT_NO_LAUNCH(ulysses_attention_local_split(A, B_, C, D_, nullptr, kMax, 4096, kMax, 1, 128,
                                                       1, bf, F, need, nullptr),
                         ULY_ERR_UNSUPPORTED);
    }

    // chunks, merge, gradients
    EXPECT_LAUNCH(ulysses_attention_chunk(A, B_, C, D_, fl(E), 1, 300, 200, 4, 2, 128, 500, 0, 1, bf,
                                          nullptr),
                  "chunk_bf16", 1, 300);
    EXPECT_LAUNCH(ulysses_attention_chunk_accumulate(A, B_, C, D_, fl(E), 1, 300, 200, 4, 2, 128, 0,
                                                     500, 1, bf, nullptr),
                  "chunk_bf16", 1, 300);
    EXPECT_NO_LAUNCH(ulysses_attention_chunk(A, B_, C, D_, fl(E), 1, 300, 200, 4, 2, 128, kMax,
                                             -kMax, 1, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_attention_chunk(A, B_, C, D_, fl(E), kMax, kMax, kMax, kMax, 1, 128, 0,
                                             0, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_LAUNCH(ulysses_attention_merge(A, fl(B_), C, fl(D_), E, fl(F), 2, 50, 4, 128, bf, nullptr),
                  "merge", 2, 50);
    EXPECT_LAUNCH(ulysses_attention_merge(A, fl(B_), C, fl(D_), A, fl(B_), 2, 50, 4, 128, bf, nullptr),
                  "merge", 2, 50);  // in place
    EXPECT_NO_LAUNCH(ulysses_attention_merge(A, fl(B_), C, fl(D_), E, fl(F), kMax, kMax, kMax, 128,
                                             bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_LAUNCH(ulysses_attention_local_backward(A, B_, C, D_, E, fl(F), fl(G), H, I, J, 1, 100, 4,
                                                   2, 128, 1, bf, nullptr),
                  "backward", 1, 100);
    EXPECT_NO_LAUNCH(ulysses_attention_local_backward(A, B_, C, D_, E, fl(F), fl(G), H, I, I, 1, 100,
                                                      4, 2, 128, 1, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_attention_local_backward(A, B_, C, D_, E, fl(F), fl(G), H, I, J, kMax,
                                                      kMax, kMax, 1, 128, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_LAUNCH(ulysses_attention_local_backward_noalloc(A, B_, C, D_, E, fl(F), H, I, J, 1, 100, 4,
                                                           2, 128, 1, bf, nullptr),
                  "backward", 1, 100);
    EXPECT_LAUNCH(ulysses_attention_local_backward_noalloc(A, B_, C, D_, E, fl(F), H, I, J, 1, 262144,
                                                           4, 4, 128, 1, bf, nullptr),
                  "backward", 1, 262144);  // exactly the scratch's 2^20 rows
    EXPECT_NO_LAUNCH(ulysses_attention_local_backward_noalloc(A, B_, C, D_, E, fl(F), H, I, J, 1,
                                                              262145, 4, 4, 128, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(ulysses_attention_local_backward_noalloc(A, B_, C, D_, E, fl(F), H, H, J, 1, 100,
                                                              4, 2, 128, 1, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_attention_local_backward_noalloc(A, B_, C, D_, E, fl(F), H, I, J, kMax,
                                                              kMax, kMax, 1, 128, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_LAUNCH(ulysses_attention_local_backward_pieces(A, B_, C, D_, E, fl(F), fl(G), H, I, J, 2, 512,
                                                          4, 2, 128, 8, 1, bf, nullptr),
                  "backward", 2, 512);
    expect(g_stub.layout == 64, "backward_pieces passes rows per piece", __LINE__);
    EXPECT_LAUNCH(ulysses_attention_local_backward(A, B_, C, D_, E, fl(F), fl(G), H, I, J, 2, 512, 4,
                                                   2, 128, 1, bf, nullptr),
                  "backward", 2, 512);
    expect(g_stub.layout == 0, "backward reads [B][S][h][D]", __LINE__);
    EXPECT_NO_LAUNCH(ulysses_attention_local_backward_pieces(A, B_, C, D_, E, fl(F), fl(G), H, I, J, 2,
                                                             96, 4, 2, 128, 3, 1, bf, nullptr),
                     ULY_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(ulysses_attention_local_backward_pieces(A, B_, C, D_, E, fl(F), fl(G), H, I, J, 2,
                                                             100, 4, 2, 128, 3, 1, bf, nullptr),
                     ULY_ERR_NOT_DIVISIBLE);
    EXPECT_NO_LAUNCH(ulysses_attention_local_backward_pieces(A, B_, C, D_, E, fl(F), fl(G), H, I, J, 2,
                                                             128, 4, 2, 128, 0, 1, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_NO_LAUNCH(ulysses_attention_local_backward_pieces(A, B_, C, D_, E, fl(F), fl(G), H, H, J, 2,
                                                             128, 4, 2, 128, 2, 1, bf, nullptr),
                     ULY_ERR_INVALID_ARGUMENT);
    EXPECT_LAUNCH(ulysses_attention_chunk_backward(A, B_, C, D_, E, fl(F), fl(G), H, I, J, 1, 300,
                                                   200, 4, 2, 128, 150, 0, 1, 0, 0, bf, nullptr),
                  "chunk_backward", 1, 300);
    EXPECT_NO_LAUNCH(ulysses_attention_chunk_backward(A, B_, C, D_, E, fl(F), fl(G), H, I, J, 1, 300,
                                                      200, 4, 2, 128, -kMax, kMax, 1, 0, 0, bf,
                                                      nullptr),
                     ULY_ERR_INVALID_ARGUMENT);

    for (int s = 0; s <= 5; ++s) expect(ulysses_status_string(uly_status_t(s)) != nullptr, "status", __LINE__);
    expect(std::strlen(ulysses_last_error()) < 512, "error string", __LINE__);
    std::printf("abi checks: %d stand-in launches, %d failures\n", g_stub.calls, failures);
    return failures ? 1 : 0;
}
