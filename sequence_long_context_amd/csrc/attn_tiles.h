// Shared pieces of the bf16 attention kernels (forward and gradients) on
// gfx950: operand types, the 64-row x 256-byte LDS tile with its XOR swizzle,
// the buffer-addressed LDS DMA that fills it, and the two ways a tile is read
// as a matrix-core A operand.  Included by attention_bf16.hip and
// attention_bwd_bf16.hip only.
#pragma once

#include "internal.h"

namespace uly {
namespace tiles {

typedef __attribute__((__vector_size__(16))) short s16x8;
typedef __attribute__((__vector_size__(8))) short s16x4;
typedef __attribute__((__vector_size__(64))) float f32x16;
typedef __attribute__((__vector_size__(16))) float f32x4;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kBN = 64;              // rows per tile
constexpr int kD = 128;              // head_dim
constexpr int kRowB = kD * 2;        // bytes per K/V row
constexpr int kTileB = kBN * kRowB;  // 16 KiB
constexpr int kStageB = 2 * kTileB;  // K tile + V tile
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ float pair_max(float x) {  // max over lanes l and l^32
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ short to_bf16(float f) {  // round to nearest even
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(short, h);
}

// LDS DMA through a buffer resource: this lane's 16 bytes at (resource base
// + voff) land at LDS byte address m0 + 16 * lane; offsets at or past the
// resource's byte count read as zero.  s_nop 4 gives the five wait states a
// vector memory instruction needs after a vector instruction wrote one of its
// scalar operands (and the one after a write of M0): the compiler's hazard
// checks do not see inside inline assembly.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16(const i32x4 &rsrc, uint32_t voff, uint32_t m0) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}
// Raw buffer resource (stride 0) over the first rows_valid rows of a tile
// whose rows are rstride elements apart: byte count (rows_valid-1)*row pitch
// + 256, so exactly the rows inside the sequence are in range.
__device__ __forceinline__ i32x4 tile_resource(const short *tile0, int rows_valid, int64_t rstride) {
    const uint64_t a = reinterpret_cast<uint64_t>(tile0);
    const uint32_t bytes = uint32_t(int64_t(rows_valid - 1) * rstride * 2 + kRowB);
    return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xFFFFu), int(bytes), 0x00020000};
}
// This wavefront's share of a 64-row tile (16 quads of 4 rows, 1 KiB each):
// quads QPW*w .. QPW*w + QPW-1 with QPW = 16 / NW; lane l of quad q lands in
// slot l%16 of row 4q + l/16 and so loads the global chunk (l%16) ^ swz(row).
template <int QPW> struct TileDma {
    uint32_t goff[QPW];  // per-lane byte offsets from the tile's first row
    uint32_t m0[QPW];    // LDS byte offsets of this wavefront's quads (uniform)
};
template <int QPW>
__device__ __forceinline__ void tile_dma_setup(TileDma<QPW> &td, int w, int lane, int64_t rstride) {
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
        const int row = (QPW * w + u) * 4 + (lane >> 4), chunk = (lane & 15) ^ swz(row);
        td.goff[u] = uint32_t(int64_t(row) * rstride * 2 + chunk * 16);
        td.m0[u] = __builtin_amdgcn_readfirstlane((QPW * w + u) * 4 * kRowB);
    }
}

__device__ __forceinline__ float bf16_to_f32(short x) {
    return __uint_as_float(uint32_t(uint16_t(x)) << 16);
}

struct LdsOff {
    int koff[8];     // A operand from tile rows (read_k form)
    int voff[2][4];  // A operand from tile columns (read_v form)
};
__device__ __forceinline__ void lds_offsets(LdsOff &f, int lane) {
    const int kr = lane & 31;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) f.koff[cc] = kr * kRowB + (((2 * cc + (lane >> 5)) ^ swz(kr)) << 4);
    const int sl = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int vr = 8 * rr + 4 * (lane >> 5) + (sl >> 2);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int dcol = 32 * mt + 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
            f.voff[rr][mt] = vr * kRowB + (((dcol >> 3) ^ swz(vr)) << 4) + ((dcol & 7) << 1);
        }
    }
}
// tile rows 32*(i&1) .. +31, columns 16*(i>>1) .. +15
__device__ __forceinline__ s16x8 rows_op(const LdsOff &f, const LDS_AS char *t, int i) {
    return *reinterpret_cast<const LDS_AS s16x8 *>(t + f.koff[i >> 1] + (i & 1) * 32 * kRowB);
}
// tile columns 32*(i&3) .. +31 as rows, tile rows 32*(i>>3) + 16*((i>>2)&1) .. +15 as k
__device__ __forceinline__ s16x8 cols_op(const LdsOff &f, const LDS_AS char *t, int i) {
    const int tt = i >> 3, h = (i >> 2) & 1, mt = i & 3;
    const int rowoff = (32 * tt + 16 * h) * kRowB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(t + f.voff[0][mt] + rowoff));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(t + f.voff[1][mt] + rowoff));
    return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// this lane's row (lane % 32) of a [rows][128] bf16 matrix as 8 B operands
__device__ __forceinline__ void load_row_operand(s16x8 (&r)[8], const short *row, int lane) {
    const short *p = row + 8 * (lane >> 5);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) r[cc] = *reinterpret_cast<const s16x8 *>(p + 16 * cc);
}
// 32x32 accumulators (4 blocks of 32 columns; lane: column l%32) scaled, to
// bf16, into row (lane % 32) of a [rows][128] matrix
__device__ __forceinline__ void store_acc_row(short *row, const f32x16 (&a)[4], float scale, int lane) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            s16x4 pv;
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = to_bf16(a[mt][4 * g + i] * scale);
            *reinterpret_cast<s16x4 *>(row + 32 * mt + 8 * g + 4 * (lane >> 5)) = pv;
        }
}

}  // namespace tiles
}  // namespace uly
