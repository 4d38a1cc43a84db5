"""C-ABI contract checks that need no GPU.

The library loads on a host without a GPU; every argument check returns
before any HIP call, so each error path can be exercised here with dummy
(never dereferenced) addresses.
"""
import os
import re
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulysses.h")

uly = pytest.importorskip("sequence_long_context_amd.ulysses")
lib = uly.library()

A = 0x7F0000000000  # dummy device addresses, 256-byte aligned, far apart
Bp = 0x7F1000000000
Cp = 0x7F2000000000
Dp = 0x7F3000000000
BF16, FP32 = uly.ULY_DTYPE_BF16, uly.ULY_DTYPE_FP32


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(ulysses_\w+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(uly.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", uly.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(r"\bT %s$" % n, out, re.M), n


def s2h(src, dst, B, S, H, D, P, dt=BF16):
    return lib.ulysses_seq_to_head(src, dst, B, S, H, D, P, dt, None)


def h2s(src, dst, B, S, H, D, P, dt=BF16):
    return lib.ulysses_head_to_seq(src, dst, B, S, H, D, P, dt, None)


def att(q, k, v, o, B, S, Hq, Hkv, D, causal=1, dt=BF16):
    return lib.ulysses_attention_local(q, k, v, o, B, S, Hq, Hkv, D, causal, dt, None)


def err():
    return lib.ulysses_last_error().decode()


@pytest.mark.parametrize("fn", [s2h, h2s])
def test_layout_errors(fn):
    assert fn(A, Bp, 1, 30, 32, 128, 8) == uly.ULY_ERR_NOT_DIVISIBLE and "S=30" in err()
    assert fn(A, Bp, 1, 32, 12, 128, 8) == uly.ULY_ERR_NOT_DIVISIBLE and "n_heads=12" in err()
    assert fn(A, Bp, 1, 64, 4, 128, 8) == uly.ULY_ERR_NOT_DIVISIBLE and "head-count" in err()
    assert fn(A, Bp, 1, 32, 32, 128, 0) == uly.ULY_ERR_INVALID_ARGUMENT
    assert fn(A, Bp, -1, 32, 32, 128, 8) == uly.ULY_ERR_INVALID_ARGUMENT
    assert fn(A, Bp, 1, -8, 32, 128, 8) == uly.ULY_ERR_INVALID_ARGUMENT
    assert fn(A, Bp, 1, 32, 32, 0, 8) == uly.ULY_ERR_INVALID_ARGUMENT
    assert fn(None, Bp, 1, 32, 32, 128, 8) == uly.ULY_ERR_INVALID_ARGUMENT and "NULL" in err()
    assert fn(A, None, 1, 32, 32, 128, 8) == uly.ULY_ERR_INVALID_ARGUMENT
    assert fn(A + 1, Bp, 1, 32, 32, 128, 8) == uly.ULY_ERR_INVALID_ARGUMENT and "aligned" in err()
    assert fn(A + 2, Bp, 1, 32, 32, 128, 8, FP32) == uly.ULY_ERR_INVALID_ARGUMENT
    # overlap: 32*32*128*2 bytes = 256 KiB; destination starts inside the source
    assert fn(A, A + 4096, 1, 32, 32, 128, 8) == uly.ULY_ERR_INVALID_ARGUMENT and "overlap" in err()
    assert fn(A, Bp, 1, 32, 32, 128, 8, 7) == uly.ULY_ERR_INVALID_ARGUMENT and "dtype" in err()
    assert fn(A, Bp, 40000, 32, 32, 128, 8) == uly.ULY_ERR_UNSUPPORTED and "P*B" in err()
    assert fn(A, Bp, 1, 1 << 40, 32, 1 << 30, 8) == uly.ULY_ERR_UNSUPPORTED


@pytest.mark.parametrize("fn", [s2h, h2s])
def test_layout_empty_is_ok_without_launch(fn):
    assert fn(None, None, 0, 32, 32, 128, 8) == uly.ULY_OK
    assert fn(None, None, 1, 0, 32, 128, 8) == uly.ULY_OK
    assert err() == ""


def test_attention_errors():
    assert att(A, Bp, Cp, Dp, 1, 64, 4, 3, 128) == uly.ULY_ERR_NOT_DIVISIBLE
    assert att(A, Bp, Cp, Dp, 1, 64, 4, 4, 64) == uly.ULY_ERR_UNSUPPORTED and "head_dim 64" in err()
    assert att(A, Bp, Cp, Dp, 1, 64, 4, 4, 48, dt=FP32) == uly.ULY_ERR_UNSUPPORTED
    assert att(A, Bp, Cp, Dp, 1, 64, 0, 1, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert att(A, Bp, Cp, Dp, -1, 64, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert att(A, Bp, Cp, None, 1, 64, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert att(A + 8, Bp, Cp, Dp, 1, 64, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    # output inside q
    assert att(A, Bp, Cp, A + 256, 1, 64, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert "overlaps" in err()
    assert att(A, Bp, Cp, Dp, 1, 1 << 31, 1, 1, 128) == uly.ULY_ERR_UNSUPPORTED
    # bf16 key/value tiles are addressed with 32-bit lane offsets
    assert att(A, Bp, Cp, Dp, 1, 64, 65537, 65537, 128) == uly.ULY_ERR_UNSUPPORTED
    assert "n_kv_heads" in err()
    assert att(A, Bp, Cp, Dp, 1, 64, 4, 4, 128, dt=9) == uly.ULY_ERR_INVALID_ARGUMENT


def test_attention_empty_is_ok_without_launch():
    assert att(None, None, None, None, 0, 64, 4, 4, 128) == uly.ULY_OK
    assert att(None, None, None, None, 1, 0, 4, 4, 128) == uly.ULY_OK


Ep, Fp, Gp, Hp, Ip, Jp = (0x7F4000000000 + i * 0x1000000000 for i in range(6))


def lse_call(q, k, v, o, lse, B, S, Hq, Hkv, D, causal=1, dt=BF16):
    return lib.ulysses_attention_local_lse(q, k, v, o, lse, B, S, Hq, Hkv, D, causal, dt, None)


def bwd(B, S, Hq, Hkv, D, ptrs=None, dt=BF16, causal=1):
    p = ptrs or [A, Bp, Cp, Dp, Ep, Fp, Gp, Hp, Ip, Jp]
    return lib.ulysses_attention_local_backward(*p, B, S, Hq, Hkv, D, causal, dt, None)


def test_lse_errors():
    assert lse_call(A, Bp, Cp, Dp, None, 1, 64, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert "lse" in err()
    assert lse_call(A, Bp, Cp, Dp, Ep + 2, 1, 64, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    # lse (4 * 64 * 4 bytes) starting inside q
    assert lse_call(A, Bp, Cp, Dp, A + 64, 1, 64, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert lse_call(A, Bp, Cp, Dp, Ep, 1, 64, 4, 3, 128) == uly.ULY_ERR_NOT_DIVISIBLE
    assert lse_call(None, None, None, None, None, 0, 64, 4, 4, 128) == uly.ULY_OK


def test_backward_errors():
    assert bwd(1, 64, 4, 4, 32, dt=FP32) == uly.ULY_ERR_UNSUPPORTED and "BF16" in err()
    assert bwd(1, 64, 4, 4, 64) == uly.ULY_ERR_UNSUPPORTED
    assert bwd(1, 64, 4, 3, 128) == uly.ULY_ERR_NOT_DIVISIBLE
    assert bwd(1, 64, 65540, 65540, 128) == uly.ULY_ERR_UNSUPPORTED
    assert bwd(-1, 64, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    for i in range(10):  # each pointer NULL in turn
        p = [A, Bp, Cp, Dp, Ep, Fp, Gp, Hp, Ip, Jp]
        p[i] = None
        assert bwd(1, 64, 4, 4, 128, p) == uly.ULY_ERR_INVALID_ARGUMENT and "NULL" in err()
    p = [A, Bp, Cp, Dp, Ep, Fp, Gp, Hp + 8, Ip, Jp]  # dq misaligned
    assert bwd(1, 64, 4, 4, 128, p) == uly.ULY_ERR_INVALID_ARGUMENT and "aligned" in err()
    p = [A, Bp, Cp, Dp, Ep, Fp, Gp, A + 1024, Ip, Jp]  # dq inside q
    assert bwd(1, 64, 4, 4, 128, p) == uly.ULY_ERR_INVALID_ARGUMENT and "overlaps an input" in err()
    p = [A, Bp, Cp, Dp, Ep, Fp, Gp, Hp, Hp + 1024, Jp]  # dk inside dq
    assert bwd(1, 64, 4, 4, 128, p) == uly.ULY_ERR_INVALID_ARGUMENT and "two outputs" in err()
    p = [A, Bp, Cp, Dp, Ep, Fp, Fp + 16, Hp, Ip, Jp]  # delta inside lse
    assert bwd(1, 64, 4, 4, 128, p) == uly.ULY_ERR_INVALID_ARGUMENT
    assert bwd(0, 64, 4, 4, 128, [None] * 10) == uly.ULY_OK


def s2h3(B, S, Hq, Hkv, D, P, ptrs=None, dt=BF16):
    p = ptrs or [A, Bp, Cp, Dp, Ep, Fp]
    return lib.ulysses_seq_to_head_qkv(*p, B, S, Hq, Hkv, D, P, dt, None)


def test_qkv_layout_errors():
    assert s2h3(1, 30, 32, 8, 128, 8) == uly.ULY_ERR_NOT_DIVISIBLE and "S=30" in err()
    assert s2h3(1, 32, 32, 4, 128, 8) == uly.ULY_ERR_NOT_DIVISIBLE and "head-count" in err()
    assert s2h3(1, 32, 32, 12, 128, 8) == uly.ULY_ERR_NOT_DIVISIBLE
    for i in range(6):
        p = [A, Bp, Cp, Dp, Ep, Fp]
        p[i] = None
        assert s2h3(1, 32, 32, 8, 128, 8, p) == uly.ULY_ERR_INVALID_ARGUMENT and "NULL" in err()
    # k_head inside q_seq
    assert s2h3(1, 32, 32, 8, 128, 8, [A, Bp, Cp, Dp, A + 4096, Fp]) == uly.ULY_ERR_INVALID_ARGUMENT
    assert "overlap" in err()
    # v_head inside q_head
    assert s2h3(1, 32, 32, 8, 128, 8, [A, Bp, Cp, Dp, Ep, Dp + 4096]) == uly.ULY_ERR_INVALID_ARGUMENT
    assert "two destinations" in err()
    assert s2h3(0, 32, 32, 8, 128, 8, [None] * 6) == uly.ULY_OK


def test_status_strings():
    assert uly.status_string(uly.ULY_OK) == "ok"
    assert uly.status_string(uly.ULY_ERR_NOT_DIVISIBLE) == "not divisible"
    assert uly.status_string(uly.ULY_ERR_HIP) == "HIP error"
    assert uly.status_string(99) == "unknown status"


def test_error_text_is_per_thread():
    import threading
    assert s2h(A, Bp, 1, 30, 32, 128, 8) == uly.ULY_ERR_NOT_DIVISIBLE
    seen = []
    t = threading.Thread(target=lambda: seen.append(err()))
    t.start()
    t.join()
    assert seen == [""] and "S=30" in err()


def test_fast_division_host(tmp_path):
    """The index decomposition's multiply-shift division is exact (host build of the same header)."""
    src = tmp_path / "fd.cpp"
    src.write_text(textwrap.dedent("""
        #include "%s"
        #include <cstdio>
        #include <random>
        int main() {
            std::mt19937_64 g(1);
            const uint32_t ds[] = {1u, 2u, 3u, 5u, 7u, 64u, 100u, 4096u, 32768u, 65535u,
                                   1u << 31, (1u << 31) + 1u, 0xFFFFFFFFu, 0xFFFFFFFEu};
            long bad = 0;
            for (uint32_t d : ds) {
                uly::FastDiv f(d);
                const uint32_t ns[] = {0u, 1u, d - 1u, d, d + 1u, 0xFFFFFFFFu, 0xFFFFFFFEu};
                for (uint32_t n : ns) bad += f.div(n) != n / d;
                for (int i = 0; i < 200000; ++i) { uint32_t n = uint32_t(g()); bad += f.div(n) != n / d; }
            }
            for (int i = 0; i < 200000; ++i) {
                uint32_t d = uint32_t(g() >> (g() %% 32)); if (!d) d = 1;
                uint32_t n = uint32_t(g());
                bad += uly::FastDiv(d).div(n) != n / d;
            }
            printf("%%ld\\n", bad);
            return bad != 0;
        }
    """ % os.path.join(ROOT, "sequence_long_context_amd", "csrc", "internal.h")))
    exe = tmp_path / "fd"
    subprocess.run(["hipcc", "-O2", "--offload-arch=gfx950", str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "0"


def chunk(q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, qp=0, kp=0, causal=1, dt=BF16):
    return lib.ulysses_attention_chunk(q, k, v, o, lse, B, Sq, Skv, Hq, Hkv, D, qp, kp, causal, dt,
                                       None)


def test_chunk_errors():
    ok = (A, Bp, Cp, Dp, Ep)
    assert chunk(*ok, 1, 64, 32, 4, 3, 128) == uly.ULY_ERR_NOT_DIVISIBLE
    assert chunk(*ok, 1, 64, 32, 4, 4, 64) == uly.ULY_ERR_UNSUPPORTED and "head_dim 64" in err()
    assert chunk(*ok, 1, -1, 32, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert chunk(*ok, 1, 64, -1, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert chunk(*ok, 1, 1 << 30, 32, 1, 1, 128) == uly.ULY_ERR_UNSUPPORTED and "2^30" in err()
    assert chunk(*ok, 1, 64, 1 << 30, 1, 1, 128) == uly.ULY_ERR_UNSUPPORTED
    assert chunk(*ok, 1, 64, 32, 4, 4, 128, qp=(1 << 62) + 1) == uly.ULY_ERR_INVALID_ARGUMENT
    assert "positions" in err()
    assert chunk(A, Bp, Cp, Dp, None, 1, 64, 32, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert "NULL" in err()
    assert chunk(A, None, Cp, Dp, Ep, 1, 64, 32, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert chunk(A + 8, Bp, Cp, Dp, Ep, 1, 64, 32, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert chunk(A, Bp, Cp, Dp, Ep + 2, 1, 64, 32, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    # o inside k; lse inside o
    assert chunk(A, Bp, Cp, Bp + 512, Ep, 1, 64, 32, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert "overlaps" in err()
    assert chunk(A, Bp, Cp, Dp, Dp + 64, 1, 64, 32, 4, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert chunk(*ok, 1, 64, 32, 4, 4, 128, dt=9) == uly.ULY_ERR_INVALID_ARGUMENT


def test_chunk_empty_is_ok_without_launch():
    assert chunk(None, None, None, None, None, 0, 64, 32, 4, 4, 128) == uly.ULY_OK
    assert chunk(None, None, None, None, None, 1, 0, 32, 4, 4, 128) == uly.ULY_OK
    assert err() == ""


def merge(oa, la, ob, lb, o, lse, B, S, H, D, dt=BF16):
    return lib.ulysses_attention_merge(oa, la, ob, lb, o, lse, B, S, H, D, dt, None)


def test_merge_errors():
    ok = (A, Bp, Cp, Dp, Ep, Fp)
    assert merge(*ok, 1, 64, 4, 96) == uly.ULY_ERR_UNSUPPORTED and "power of two" in err()
    assert merge(*ok, 1, 64, 4, 4) == uly.ULY_ERR_UNSUPPORTED  # 8 bytes per row
    assert merge(*ok, 1, 64, 4, 1024) == uly.ULY_ERR_UNSUPPORTED  # 2048 bytes per row
    assert merge(*ok, 1, 64, 4, 2, dt=FP32) == uly.ULY_ERR_UNSUPPORTED
    assert merge(*ok, 1 << 16, 1 << 16, 1, 128) == uly.ULY_ERR_UNSUPPORTED and "2^32" in err()
    assert merge(*ok, -1, 64, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert merge(*ok, 1, 64, 0, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert merge(*ok, 1, 64, 4, 128, dt=5) == uly.ULY_ERR_INVALID_ARGUMENT
    for i in range(6):
        p = list(ok)
        p[i] = None
        assert merge(*p, 1, 64, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT and "NULL" in err()
    assert merge(A + 8, Bp, Cp, Dp, Ep, Fp, 1, 64, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert merge(A, Bp + 2, Cp, Dp, Ep, Fp, 1, 64, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    # o partly overlapping o_a; lse partly overlapping lse_b; o over lse_a
    assert merge(A, Bp, Cp, Dp, A + 256, Fp, 1, 64, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert merge(A, Bp, Cp, Dp, Ep, Dp + 16, 1, 64, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT
    assert merge(A, Bp, Cp, Dp, Bp, Fp, 1, 64, 4, 128) == uly.ULY_ERR_INVALID_ARGUMENT


def test_merge_empty_is_ok_without_launch():
    assert merge(None, None, None, None, None, None, 0, 64, 4, 128) == uly.ULY_OK
    assert merge(None, None, None, None, None, None, 1, 0, 4, 128) == uly.ULY_OK
    assert err() == ""


def test_chunk_accumulate_errors():
    f = lib.ulysses_attention_chunk_accumulate
    assert f(A, Bp, Cp, Dp, Ep, 1, 64, 32, 4, 4, 32, 0, 0, 1, FP32, None) == uly.ULY_ERR_UNSUPPORTED
    assert "BF16" in err()
    assert f(A, Bp, Cp, Dp, None, 1, 64, 32, 4, 4, 128, 0, 0, 1, BF16, None) == uly.ULY_ERR_INVALID_ARGUMENT
    assert f(A, Bp, Cp, Dp, Dp + 64, 1, 64, 32, 4, 4, 128, 0, 0, 1, BF16, None) == uly.ULY_ERR_INVALID_ARGUMENT
    assert f(None, None, None, None, None, 1, 0, 32, 4, 4, 128, 0, 0, 1, BF16, None) == uly.ULY_OK


def chunk_bwd(B, Sq, Skv, Hq, Hkv, D, ptrs=None, dt=BF16, qp=0, kp=0):
    p = ptrs or [A, Bp, Cp, Dp, Ep, Fp, Gp, Hp, Ip, Jp]
    return lib.ulysses_attention_chunk_backward(*p, B, Sq, Skv, Hq, Hkv, D, qp, kp, 1, 0, 0, dt, None)


def test_chunk_backward_errors():
    assert chunk_bwd(1, 64, 32, 4, 4, 32, dt=FP32) == uly.ULY_ERR_UNSUPPORTED and "BF16" in err()
    assert chunk_bwd(1, 64, 32, 4, 3, 128) == uly.ULY_ERR_NOT_DIVISIBLE
    assert chunk_bwd(1, 1 << 30, 32, 1, 1, 128) == uly.ULY_ERR_UNSUPPORTED and "2^30" in err()
    assert chunk_bwd(1, 64, 32, 4, 4, 128, qp=-(1 << 62) - 1) == uly.ULY_ERR_INVALID_ARGUMENT
    for i in range(10):  # each pointer NULL in turn
        p = [A, Bp, Cp, Dp, Ep, Fp, Gp, Hp, Ip, Jp]
        p[i] = None
        assert chunk_bwd(1, 64, 32, 4, 4, 128, p) == uly.ULY_ERR_INVALID_ARGUMENT and "NULL" in err()
    # dq (index 7) inside q
    p = [A, Bp, Cp, Dp, Ep, Fp, Gp, A + 256, Ip, Jp]
    assert chunk_bwd(1, 64, 32, 4, 4, 128, p) == uly.ULY_ERR_INVALID_ARGUMENT and "overlaps" in err()
    assert chunk_bwd(0, 64, 32, 4, 4, 128, [None] * 10) == uly.ULY_OK
