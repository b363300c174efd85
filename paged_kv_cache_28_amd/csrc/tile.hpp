// One (block, KV head) tile of K and V as a lane holds it for the two matrix products of
// the decode kernels, the operands taken from it, and row masking. The 16 columns of both
// products are the query heads of a GQA group. The prefill kernel walks keys in 32-position
// pairs of its own layout and takes only q_dim from here (its Q^T operand order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace pkv {

// K and V of one (block, KV head) tile as this lane holds them for the two products,
// per cache type, and the operands the matrix instructions take from it.
//   16-bit cache: k[c] is the A operand of QK step c (dims 32c + 8 quad .. + 7 of token
//     l%16, 16 bytes at (64c + l) * 16 of the [d/8][16][8] tile); v[c] that of PV step c
//     (dim 16c + l%16, tokens 4 quad .. + 3).
//   FP8 cache ([d/16][16][16] bytes): one 16-byte load k[i] at (64i + l) * 16 holds dims
//     16(4i + quad) .. + 15 of token l%16 and feeds QK steps 2i (its first 8 dims) and
//     2i + 1 (the last 8); the dimensions of the contraction are taken in another order,
//     and the Q^T operand follows the same order (q_dim). v[c] holds the four codes of
//     PV step c. The codes are widened to T when used.
template <int D, bool F8> struct KvTile;
template <int D> struct KvTile<D, false> {
    uint4 k[D / 32];
    uint2 v[D / 16];
};
template <int D> struct KvTile<D, true> {
    uint4 k[D / 64];
    uint32_t v[D / 16];
};

// First query dimension of the 8 that lane group `quad` feeds QK step c with.
template <bool F8>
__device__ __forceinline__ int q_dim(int c, int quad) {
    return F8 ? 64 * (c >> 1) + 16 * quad + 8 * (c & 1) : 32 * c + 8 * quad;
}

// Cache policy of the tile loads: non-temporal, except for the half-block tiles of 32-token
// blocks, whose K and V lines hold rows of both halves, which two waves read at about the
// same time (non-temporal loads there made the 8B batch at 32 tokens per block 11% slower
// in the single pass and 17% in the balanced split).
template <int BS>
constexpr int kTilePol = BS == 32 ? 0 : kBufNT;

// Loads of one 16-token tile, through buffer resources over the (block, KV head) tiles
// (tile_rsrc): ka/va cover the tile of block A; for BS = 32, row0 (0 or 16) picks the
// half, added as a scalar offset (BS = 16 ignores it: the tile is the block). BS = 8 takes
// rows 0-7 from block A and 8-15 from block B, a choice that differs between lanes, so it
// reads through per-lane addresses instead.
template <int D, int BS>
__device__ __forceinline__ void load_tile_bs(KvTile<D, false>& t, const char* ka, const char* va,
                                             const char* kb, const char* vb, int row0, int lane) {
    static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
    const int col = lane & 15, quad = lane >> 4;
    if constexpr (BS == 8) {
        const char* kt = col < 8 ? ka : kb;
        const int krow = col & 7;
        const char* vt = quad < 2 ? va : vb;
        const int vrow = 4 * (quad & 1);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) t.k[c] = ld_once16(kt + ((4 * c + quad) * BS + krow) * 16);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) t.v[c] = ld_once8(vt + ((16 * c + col) * BS + vrow) * 2);
    } else {
        const int r0 = BS == 32 ? row0 : 0;
        const buf_rsrc_t kr = tile_rsrc(ka, D * BS * 2), vr = tile_rsrc(va, D * BS * 2);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) t.k[c] = bld16<kTilePol<BS>>(kr, ((4 * c + quad) * BS + col) * 16, r0 * 16);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) t.v[c] = bld8<kTilePol<BS>>(vr, ((16 * c + col) * BS + 4 * quad) * 2, r0 * 2);
    }
}
template <int D, int BS>
__device__ __forceinline__ void load_tile_bs(KvTile<D, true>& t, const char* ka, const char* va,
                                             const char* kb, const char* vb, int row0, int lane) {
    static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
    const int col = lane & 15, quad = lane >> 4;
    if constexpr (BS == 8) {
        const char* kt = col < 8 ? ka : kb;
        const int krow = col & 7;
        const char* vt = quad < 2 ? va : vb;
        const int vrow = 4 * (quad & 1);
#pragma unroll
        for (int i = 0; i < D / 64; ++i) t.k[i] = ld_once16(kt + ((4 * i + quad) * BS + krow) * 16);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) t.v[c] = ld_once4(vt + (16 * c + col) * BS + vrow);
    } else {
        const int r0 = BS == 32 ? row0 : 0;
        const buf_rsrc_t kr = tile_rsrc(ka, D * BS), vr = tile_rsrc(va, D * BS);
#pragma unroll
        for (int i = 0; i < D / 64; ++i) t.k[i] = bld16<kTilePol<BS>>(kr, ((4 * i + quad) * BS + col) * 16, r0 * 16);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) t.v[c] = bld4<kTilePol<BS>>(vr, (16 * c + col) * BS + 4 * quad, r0);
    }
}

// Block ids behind 16-token tile t of a block-table row with max_blocks entries: ida is
// the block holding the tile's rows 0-7 (all 16 when BS >= 16), idb the one holding rows
// 8-15 when BS = 8 (else -1); an index past the row gives -1.
template <int BS>
__device__ __forceinline__ void tile_ids(const int32_t* row, int max_blocks, int t, int& ida,
                                         int& idb) {
    if constexpr (BS == 8) {
        ida = 2 * t < max_blocks ? row[2 * t] : -1;
        idb = 2 * t + 1 < max_blocks ? row[2 * t + 1] : -1;
    } else {
        const int i = BS == 32 ? t >> 1 : t;
        ida = i < max_blocks ? row[i] : -1;
        idb = -1;
    }
}

template <typename T, int D>
__device__ __forceinline__ uint4 k_operand(const KvTile<D, false>& t, int c) { return t.k[c]; }
template <typename T, int D>
__device__ __forceinline__ uint4 k_operand(const KvTile<D, true>& t, int c) {
    const uint4 w = t.k[c >> 1];
    const uint2 a = Fp8<T>::x4((c & 1) ? w.z : w.x), b = Fp8<T>::x4((c & 1) ? w.w : w.y);
    return make_uint4(a.x, a.y, b.x, b.y);
}
template <typename T, int D>
__device__ __forceinline__ uint2 v_operand(const KvTile<D, false>& t, int c) { return t.v[c]; }
template <typename T, int D>
__device__ __forceinline__ uint2 v_operand(const KvTile<D, true>& t, int c) { return Fp8<T>::x4(t.v[c]); }

// Zero V rows tok0 + e (e = 0..3) of this lane whose keep[e] is false, so that whatever
// bytes a partly filled block holds there never reach the sum (0 weight times NaN would).
template <int D>
__device__ __forceinline__ void mask_rows(KvTile<D, false>& t, bool k0, bool k1, bool k2, bool k3) {
    const uint32_t lo = (k0 ? 0x0000ffffu : 0u) | (k1 ? 0xffff0000u : 0u);
    const uint32_t hi = (k2 ? 0x0000ffffu : 0u) | (k3 ? 0xffff0000u : 0u);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        t.v[c].x &= lo;
        t.v[c].y &= hi;
    }
}
template <int D>
__device__ __forceinline__ void mask_rows(KvTile<D, true>& t, bool k0, bool k1, bool k2, bool k3) {
    const uint32_t m = (k0 ? 0xffu : 0u) | (k1 ? 0xff00u : 0u) | (k2 ? 0xff0000u : 0u) |
                       (k3 ? 0xff000000u : 0u);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) t.v[c] &= m;
}

}  // namespace pkv
