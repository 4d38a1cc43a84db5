// Sequence-shard <-> head-shard layout change of DeepSpeed-Ulysses, P virtual
// ranks in one HBM ("Sequence Parallelism II: DeepSpeed Ulysses and All-to-All
// Attention", sections 1 and 3; "Comparing Ulysses and Megatron Sequence
// Parallelism", section "DeepSpeed Attention").
//
// One source token row SEQ[i][b][t][:][:] is H*D elements; it splits into P
// runs of (H/P)*D contiguous elements, run j landing contiguously at
// HEAD[j][b][i*S/P + t][:][:].  head_dim is innermost on both sides, so the
// whole exchange (pack, the virtual send, unpack) is one pass of contiguous
// run copies: no element-level transpose exists in this layout, and every
// wavefront touches whole 128-byte-or-longer runs on both the read and the
// write side.  The kernel walks one side linearly, one 16-byte vector per
// thread, and computes the matching address on the other: the SEQ side
// (grid.y = (source rank i, batch b), grid.x = the vectors of that rank's
// token rows), or for seq -> head with runs of at most 512 bytes the HEAD side
// (grid.y = (destination rank j, batch b), grid.x = the vectors of the rows it
// receives), so that the short runs are read and the writes are contiguous.
// Measured on MI355X, seq -> head of one 32-head bf16 tensor: 256-byte runs
// (262144 tokens, P = 32) 5751 -> 6061 GB/s walking the HEAD side, 512-byte
// runs (P = 16) 5842 -> 6242, 256-byte runs (65536 tokens, 8 heads, P = 8)
// 6014 -> 6243; 1 KiB runs (32768 tokens, P = 8) 6572 walking SEQ against
// 6444.  Among SEQ-order walks, one vector per thread measured fastest against
// 2-16 vectors per thread and 128-1024 threads per block.
//
// The head side has two layouts.  HEAD[j][b][i*S/P + t] stacks the pieces a
// rank receives along the sequence, per batch entry.  PIECES[j][i][b][t]
// keeps them in the order the exchange delivers them (one [B][S/P] piece from
// every source rank i, "Sequence Parallelism II...", section 3): the receive
// buffer of the first exchange before any unpack, and the send buffer of the
// second.  The two differ only for B > 1; a head-side token row (j, i, b, t)
// sits at row j*B*S + i*peer_rows + b*batch_rows + t of the buffer, with
// (peer_rows, batch_rows) = (S/P, S) for HEAD and (B*S/P, S/P) for PIECES.
//
// Per element the algorithmic traffic is one read and one write (2 * elem
// bytes); the kernel is bound by HBM bandwidth.  Loads are marked
// non-temporal: every source byte is read once.  Stores are 16-byte buffer
// stores at device scope (sc1): each XCD writes them through its own L2, so
// no dirty lines are left for a write-back later, and what fits stays in the
// memory-side cache for the attention that reads the head side next.  Measured
// on MI355X over the step (seq -> head of Q, K and V in one launch, one rank's
// attention, head -> seq of O; 32 heads, P = 8), against regular stores on the
// head side and non-temporal ones on the sequence side: S = 32768 Q/K/V
// exchange 251.1 -> 239.1 us, O exchange 85.9 -> 76.0 us; S = 4096 37.1 ->
// 35.0 and 15.4 -> 13.4 us; the attentions after them unchanged.  (Before
// that, non-temporal stores on the head side had cost the S = 4096 attention
// 62.6 against 47.5 us: they send the output past the memory-side cache.)
// Destinations of 4 GiB or more, and vectors narrower than 16 bytes, keep
// regular stores on the head side and non-temporal ones on the sequence side.
#include "internal.h"

namespace uly {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int VB> struct VecT;
template <> struct VecT<16> { typedef u32x4 type; };
template <> struct VecT<8> { typedef u32x2 type; };
template <> struct VecT<4> { typedef unsigned int type; };
template <> struct VecT<2> { typedef unsigned short type; };
template <> struct VecT<1> { typedef unsigned char type; };

constexpr int kThreads = 256;

struct LayoutArgs {
    const void *src;
    void *dst;
    uint32_t slice_vecs;  // (S/P) * P * W: vectors of one (source rank i, batch b) SEQ slice
    uint32_t Sp;          // tokens per rank
    uint32_t B;
    uint32_t S;
    uint32_t peer_rows;   // head-side rows between the pieces of source ranks i and i + 1
    uint32_t batch_rows;  // head-side rows between batch entries b and b + 1
    FastDiv by_W;         // W = vectors per run ((H/P)*D*elem / VB)
    FastDiv by_PW;        // P * W = vectors per token row
    FastDiv by_Sp;        // S/P
    uint32_t headwalk;    // seq -> head walking the HEAD side (grid.y = (j, b))
    uint32_t dst_bytes;   // destination size when below 4 GiB (device-scope stores), else 0
};

// 16-byte store of vector idx of dst at device scope (sc1), through a buffer
// resource over the dst_bytes bytes of the destination
__device__ __forceinline__ void store_device16(void *dst, uint32_t dst_bytes, uint64_t idx, u32x4 val) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, int(dst_bytes), 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, val), rs, int(uint32_t(idx * 16u)), 0, 16);
}

// SEQ and HEAD vector indices of vector u of grid row y.  SEQ walk: y = i*B + b
// and u runs over rank i's token rows (token t, then run j, then vector w);
// HEAD walk: y = j*B + b and u runs over the rows rank j receives (row s =
// i*S/P + t, then vector w).
__device__ __forceinline__ void layout_index(const LayoutArgs &a, uint32_t y, uint32_t u,
                                             uint64_t &seq_idx, uint64_t &head_idx) {
    const uint32_t W = a.by_W.d;
    const uint32_t r = y / a.B, b = y - r * a.B;
    uint32_t i, j, t, w;
    if (a.headwalk) {
        const uint32_t s = a.by_W.div(u);
        w = u - s * W;
        j = r;
        i = a.by_Sp.div(s);
        t = s - i * a.Sp;
    } else {
        t = a.by_PW.div(u);
        const uint32_t rem = u - t * a.by_PW.d;
        j = a.by_W.div(rem);
        w = rem - j * W;
        i = r;
    }
    seq_idx = ((uint64_t(i) * a.B + b) * a.Sp + t) * a.by_PW.d + uint64_t(j) * W + w;
    head_idx = (uint64_t(j) * a.B * a.S + uint64_t(i) * a.peer_rows + uint64_t(b) * a.batch_rows + t) * W + w;
}

template <int VB, bool TO_HEAD>
__global__ __launch_bounds__(kThreads) void layout_kernel(LayoutArgs a) {
    typedef typename VecT<VB>::type V;
    const uint32_t u = blockIdx.x * kThreads + threadIdx.x;  // vector inside the walked slice
    if (u >= a.slice_vecs) return;
    uint64_t seq_idx, head_idx;
    layout_index(a, blockIdx.y, u, seq_idx, head_idx);
    const V *src = static_cast<const V *>(a.src);
    V *dst = static_cast<V *>(a.dst);
    const V val = __builtin_nontemporal_load(src + (TO_HEAD ? seq_idx : head_idx));
    if constexpr (VB == 16) {
        if (a.dst_bytes) {
            store_device16(a.dst, a.dst_bytes, TO_HEAD ? head_idx : seq_idx, val);
            return;
        }
    }
    if (TO_HEAD)
        dst[head_idx] = val;
    else
        __builtin_nontemporal_store(val, dst + seq_idx);
}

// Q, K and V in one launch: grid.x is the blocks of Q's slice, then K's, then
// V's (first[x] = tensor x's first block), so that no block is idle when K
// and V have fewer heads than Q.  (A grid over the largest slice with
// blockIdx.z picking the tensor launches empty blocks instead: with 4 query
// heads per key head, half of the grid; measured on MI355X at 65536 tokens, 32
// query and 8 key/value heads, P = 8: 271.5 us, against 258.4 us for three
// launches.)
struct LayoutArgs3 {
    LayoutArgs t[3];
    uint32_t first[3];
};
template <int VB>
__global__ __launch_bounds__(kThreads) void layout3_kernel(LayoutArgs3 a) {
    typedef typename VecT<VB>::type V;
    const uint32_t tx = blockIdx.x >= a.first[2] ? 2u : blockIdx.x >= a.first[1] ? 1u : 0u;
    const LayoutArgs &x = a.t[tx];
    const uint32_t u = (blockIdx.x - a.first[tx]) * kThreads + threadIdx.x;
    if (u >= x.slice_vecs) return;
    uint64_t seq_idx, head_idx;
    layout_index(x, blockIdx.y, u, seq_idx, head_idx);
    const V val = __builtin_nontemporal_load(static_cast<const V *>(x.src) + seq_idx);
    if constexpr (VB == 16) {
        if (x.dst_bytes) {
            store_device16(x.dst, x.dst_bytes, head_idx, val);
            return;
        }
    }
    static_cast<V *>(x.dst)[head_idx] = val;
}

template <int VB>
hipError_t launch_vb(const LayoutArgs &a, uint32_t PB, bool to_head, hipStream_t st) {
    dim3 grid((a.slice_vecs + kThreads - 1) / kThreads, PB);
    if (to_head)
        hipLaunchKernelGGL((layout_kernel<VB, true>), grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((layout_kernel<VB, false>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

namespace {
LayoutArgs make_args(const void *src, void *dst, int64_t B, int64_t S, int64_t H, int64_t D,
                     int32_t P, int vb, int32_t elem, bool pieces, bool to_head) {
    const int64_t W = (H / P) * D * elem / vb;
    LayoutArgs a;
    a.src = src;
    a.dst = dst;
    a.slice_vecs = uint32_t(S * W);  // (S/P) token rows of P runs of W vectors
    a.Sp = uint32_t(S / P);
    a.B = uint32_t(B);
    a.S = uint32_t(S);
    a.peer_rows = uint32_t(pieces ? B * (S / P) : S / P);
    a.batch_rows = uint32_t(pieces ? S / P : S);
    a.by_W = FastDiv(uint32_t(W));
    a.by_PW = FastDiv(uint32_t(P * W));
    a.by_Sp = FastDiv(uint32_t(S / P));
    // both walks cover S * W vectors per grid row
    a.headwalk = to_head && (H / P) * D * elem <= 512 ? 1u : 0u;
    const uint64_t bytes = uint64_t(B) * uint64_t(S) * uint64_t(H) * uint64_t(D) * uint64_t(elem);
    a.dst_bytes = vb == 16 && bytes < (uint64_t(1) << 32) ? uint32_t(bytes) : 0u;
    return a;
}
// One launch while the three slices' blocks together stay below 2^32 work
// items in x; past that, the three tensors' own launches.
template <int VB>
hipError_t launch3_vb(LayoutArgs3 &a, uint32_t PB, hipStream_t st) {
    uint64_t blocks = 0;
    for (int x = 0; x < 3; ++x) {
        a.first[x] = uint32_t(blocks);
        blocks += (a.t[x].slice_vecs + kThreads - 1) / kThreads;
    }
    if (blocks * kThreads >= (uint64_t(1) << 32)) {
        for (int x = 0; x < 3; ++x) {
            hipError_t err = launch_vb<VB>(a.t[x], PB, true, st);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    }
    dim3 grid(uint32_t(blocks), PB);
    hipLaunchKernelGGL((layout3_kernel<VB>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_layout_qkv(const void *const src[3], void *const dst[3], int64_t B, int64_t S,
                             int64_t Hq, int64_t Hkv, int64_t D, int32_t P, int32_t elem,
                             bool pieces, hipStream_t st) {
    // widest vector that divides every run and every base address
    uint64_t align = 16u;
    for (int x = 0; x < 3; ++x) {
        const int64_t H = x == 0 ? Hq : Hkv;
        align |= uint64_t((H / P) * D * elem) | reinterpret_cast<uintptr_t>(src[x]) |
                 reinterpret_cast<uintptr_t>(dst[x]);
    }
    const int vb = int(align & (~align + 1));
    LayoutArgs3 a;
    for (int x = 0; x < 3; ++x)
        a.t[x] = make_args(src[x], dst[x], B, S, x == 0 ? Hq : Hkv, D, P, vb, elem, pieces, true);
    const uint32_t PB = uint32_t(P * B);
    switch (vb) {
        case 16: return launch3_vb<16>(a, PB, st);
        case 8: return launch3_vb<8>(a, PB, st);
        case 4: return launch3_vb<4>(a, PB, st);
        case 2: return launch3_vb<2>(a, PB, st);
        default: return launch3_vb<1>(a, PB, st);
    }
}

hipError_t launch_layout(const void *src, void *dst, int64_t B, int64_t S, int64_t H,
                         int64_t D, int32_t P, int32_t elem, bool to_head, bool pieces,
                         hipStream_t st) {
    const int64_t run_bytes = (H / P) * D * elem;
    // widest vector that divides the run and both base addresses
    const uint64_t align = uint64_t(run_bytes) | reinterpret_cast<uintptr_t>(src) |
                           reinterpret_cast<uintptr_t>(dst) | 16u;
    const int vb = int(align & (~align + 1));  // lowest set bit, at most 16
    const LayoutArgs a = make_args(src, dst, B, S, H, D, P, vb, elem, pieces, to_head);
    const uint32_t PB = uint32_t(P * B);
    switch (vb) {
        case 16: return launch_vb<16>(a, PB, to_head, st);
        case 8: return launch_vb<8>(a, PB, to_head, st);
        case 4: return launch_vb<4>(a, PB, to_head, st);
        case 2: return launch_vb<2>(a, PB, to_head, st);
        default: return launch_vb<1>(a, PB, to_head, st);
    }
}

}  // namespace uly
