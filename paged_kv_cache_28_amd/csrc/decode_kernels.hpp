// Kernels of paged_attention_decode: single-query attention for a batch of sequences
// whose K/V live in scattered blocks of BS tokens (8, 16 or 32) reached through
// per-sequence block tables. Each block size is instantiated in a translation unit of its
// own (decode.hip: 16, decode_bs8.hip, decode_bs32.hip) through dispatch_bs.
//
// The attention math is ordinary scaled dot-product attention; paging only changes
// where K and V are read from ("vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem,
// closing paragraphs; the block table is step 2 there). Grouped-query attention lets
// the query heads of a group share one KV head ("Yerel LLM sistemlerinde backpressure
// ve ölçekleme", section "KV bütçesi"), so every KV tile is loaded once and used for
// all G = Hq / Hkv query heads of its group.
//
// Work decomposition, three launch modes:
//   single pass / fixed partitions (decode_mfma_kernel): one workgroup per (context
//     partition, KV head, sequence); its W waves take the partition's blocks
//     round-robin, each keeping its own online softmax state, and merge through LDS at
//     the end. A sequence with one partition writes its output; otherwise the partition
//     writes (o_p, m_p, l_p) for the reduce.
//   balanced split (decode_split_kernel): all tiles of the batch cut into equal runs,
//     one per wave (split.hpp); pieces that do not cover their (sequence, KV head) leave
//     records for the reduce.
//   fp32 inputs (decode_f32_kernel): plain vector arithmetic, the correctness path.
// The fused append (paged_attention_decode_append) also stores each sequence's new K/V
// row and, in the first two modes, attends to it from the key/value inputs.
//
// fp16/bf16 path, one wave per tile of 16 tokens (matrix instructions, wave64); the
// layout offsets below are those of BS = 16 (tile.hpp gives the others):
//   S^T[16 tokens][16 cols] = K_tile[16][d] x Q^T[d][16 cols]   (16x16x32, d/32 steps)
//      A = K tile: lane l holds token l%16, dims 32c + 8(l/16) .. +7. In the cache
//          layout [d/8][16][8] that is the 16 bytes at (64c + l) * 16: each step
//          reads 1 KiB contiguous.
//      B = Q^T: lane l holds query head l%16 of the group (zero past G), same dims.
//      C: lane l holds head l%16 for tokens 4(l/16) + e, e = 0..3.
//   online softmax on those 4 values (cross-lane max over lanes l^16, l^32, which
//   hold the other tokens of the same head);
//   O^T[d][16 cols] += V^T[d][16 tokens] x P^T[16 tokens][16 cols]  (16x16x16, d/16)
//      A = V^T: lane l holds dim 16c + l%16, tokens 4(l/16) + e: 8 bytes at
//          (16c + l%16) * 32 + 8 (l/16) in the [d][16] layout (512 B per step).
//      B = P^T: exactly the C layout of the first product, so no data movement.
//      P is split into a high and a low part in the input type (two products), so
//      the weights keep ~16 significant bits instead of 8 (bf16) or 11 (fp16).
//   C: lane l holds head l%16, dims 16c + 4(l/16) + e: its rescale factor is the
//      lane's own running max, so the online softmax needs no transposes.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>

#include "device.hpp"
#include "split.hpp"
#include "tile.hpp"
#include "status.hpp"
#include "timer.hpp"

namespace pkv {

constexpr int kLptMaxSeqs = 256;

// K/V tiles in flight per wave in the single-pass / partitioned kernel (1, 2 or 3).
#ifndef PKV_DECODE_BUFFERS
#define PKV_DECODE_BUFFERS 2
#endif
constexpr int kDecodeBuffers = PKV_DECODE_BUFFERS;

struct DecodeArgs {
    void* out;
    float* part_out;
    float* part_max;
    float* part_sum;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    int64_t q_stride;      // elements between sequences in q
    int64_t num_blocks;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t group;         // G = num_heads / num_kv_heads
    int32_t max_blocks;    // block-table row length
    int32_t max_len;       // max_blocks * block size: longest context the table holds
    int32_t max_tiles;     // ceil(max_len / 16): 16-token tiles of the longest context
    int32_t part_tiles;    // 16-token tiles per partition
    int32_t max_partitions;
    float scale_log2;      // scale * log2(e) (* k_scale for an FP8 cache): base-2 logits
    float k_scale;         // FP8 cache: per-tensor scales (new rows are quantised with
    float v_scale;         // them; v_scale multiplies every output); 1 otherwise
    int32_t num_seqs;
    SplitParams split;     // balanced mode only
    int32_t slots;         // balanced mode: result slots per wave
    // Grid order of the single-pass / partitioned kernels. Consecutive workgroups go to
    // different XCDs. With fewer than 8 partitions per sequence, partition-fastest order
    // would put every partition 0 on the same few XCDs, so the grid is (KV head, sequence,
    // partition); with 8 or more it is (partition, KV head, sequence), which measured
    // faster on long contexts.
    int32_t heads_fastest;
    // Fixed partitions: each wave takes a partition of its own (kWaves partitions per
    // workgroup, grid slot pg holding partitions pg kWaves ..) and writes its record, so a
    // workgroup's fixed costs (queries, block ids, the first tiles' latency, the merge) are
    // paid once per kWaves partitions rather than once per partition.
    int32_t per_wave;
    // Single pass with at most kLptMaxSeqs sequences: workgroups are dispatched one CU
    // after the other, one round of lpt_round sequences (x KV heads) per sweep over the
    // CUs, and a CU keeps the workgroups of all rounds. The sequences are handed out by
    // length in serpentine order (round 0 takes ranks 0 .. R-1, round 1 ranks 2R-1 .. R,
    // ...), so a CU that holds one of the longest also holds one of the shortest and the
    // CUs finish together. 0: sequences in index order (or in the host plan's order).
    int32_t lpt_round;
    // The same serpentine order computed on the host from a host copy of the lengths
    // (paged_attention_decode_plan, once per step for every layer): slot b of the grid takes
    // sequence order[b], so the kernel starts with its queries and block ids instead of a
    // length load and the ranking. Only used with lpt_round == 0.
    int32_t use_order;
    uint16_t order[kLptMaxSeqs];
    // fused append (paged_attention_decode_append): the new token of sequence b has
    // rows new_k/new_v + b * new_*_stride ([Hkv][D]) and goes to slot_mapping[b]
    const void* new_k;
    const void* new_v;
    const int32_t* slot_mapping;
    int64_t new_k_stride;
    int64_t new_v_stride;
};

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.44269504088896340736f;

// Write the zero row of an empty sequence (n == 0) for the G heads of group g.
template <typename OutT, int D>
__device__ void write_zero_rows(const DecodeArgs& a, int b, int g) {
    for (int i = threadIdx.x; i < a.group * D; i += blockDim.x) {
        const int h = g * a.group + i / D;
        OutStore<OutT>::st(a.out, (int64_t(b) * a.num_heads + h) * D + i % D, 0.0f);
    }
}

// Fused append: copy the new token's K and V rows of KV head g into its slot (the
// reshape_and_cache layout; FP8 cache: their codes, as reshape_and_cache_fp8 stores
// them), with the threads of the calling workgroup. A slot outside the pool (or
// negative) is skipped, as reshape_and_cache does.
template <typename T, int D, bool F8, int BS>
__device__ void write_new_token(const DecodeArgs& a, int b, int g, int slot) {
    if (slot < 0 || int64_t(slot) >= a.num_blocks * BS) return;
    const int64_t tile = int64_t(slot / BS) * a.num_kv_heads + g;
    const int off = slot % BS;
    const uint16_t* krow = static_cast<const uint16_t*>(a.new_k) + int64_t(b) * a.new_k_stride + int64_t(g) * D;
    const uint16_t* vrow = static_cast<const uint16_t*>(a.new_v) + int64_t(b) * a.new_v_stride + int64_t(g) * D;
    const int t = threadIdx.x;
    if constexpr (F8) {
        uint8_t* kc = const_cast<uint8_t*>(static_cast<const uint8_t*>(a.k_cache));
        uint8_t* vc = const_cast<uint8_t*>(static_cast<const uint8_t*>(a.v_cache));
        if (t < D / 16)   // K: [tile][d/16][BS][16] bytes, one 16-byte group per thread
            *reinterpret_cast<uint4*>(kc + ((tile * (D / 16) + t) * BS + off) * 16) =
                quantize_fp8_x16<T>(*reinterpret_cast<const uint4*>(krow + 16 * t),
                                    *reinterpret_cast<const uint4*>(krow + 16 * t + 8), a.k_scale);
        for (int d = t; d < D; d += blockDim.x)   // V: [tile][d][BS] bytes
            vc[(tile * D + d) * BS + off] = uint8_t(quantize_fp8(Bits<T>::to_f32(vrow[d]), a.v_scale));
    } else {
        uint16_t* kc = const_cast<uint16_t*>(static_cast<const uint16_t*>(a.k_cache));
        uint16_t* vc = const_cast<uint16_t*>(static_cast<const uint16_t*>(a.v_cache));
        if (t < D / 8)   // K: [tile][d/8][BS][8], one 16-byte group per thread
            *reinterpret_cast<uint4*>(kc + ((tile * (D / 8) + t) * BS + off) * 8) =
                *reinterpret_cast<const uint4*>(krow + 8 * t);
        for (int d = t; d < D; d += blockDim.x)   // V: [tile][d][BS]
            vc[(tile * D + d) * BS + off] = vrow[d];
    }
}

// FP8 fused append, in two halves. load_new_row_fp8: this lane's D/64 consecutive raw
// elements of the new K and V rows. quantize_new_row_fp8: their codes, met in the wave's
// LDS slice q8 (2 D bytes), from which every lane takes the ones it holds in the tile
// layout: nk[i] the 16 codes of K group 4 i + quad, nv[c] the code of dimension 16 c + col.
// Quantising whole K groups per lane instead cost 40 divisions per lane.
template <int D>
__device__ __forceinline__ void load_new_row_fp8(const uint16_t* krow, const uint16_t* vrow,
                                                 int lane, uint32_t& nkr, uint32_t& nvr) {
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    if constexpr (D == 128) {
        nkr = *reinterpret_cast<const uint32_t*>(krow + 2 * lane);
        nvr = *reinterpret_cast<const uint32_t*>(vrow + 2 * lane);
    } else {
        nkr = krow[lane];
        nvr = vrow[lane];
    }
}
template <typename T, int D>
__device__ __forceinline__ void quantize_new_row_fp8(const DecodeArgs& a, uint8_t* q8, int lane,
                                                     uint32_t nkr, uint32_t nvr, uint4* nk,
                                                     uint32_t* nv) {
    constexpr int NQ = D / 64;
    const int col = lane & 15, quad = lane >> 4;
#pragma unroll
    for (int e = 0; e < NQ; ++e) {
        q8[NQ * lane + e] = uint8_t(quantize_fp8(Bits<T>::to_f32(uint16_t(nkr >> (16 * e))), a.k_scale));
        q8[D + NQ * lane + e] = uint8_t(quantize_fp8(Bits<T>::to_f32(uint16_t(nvr >> (16 * e))), a.v_scale));
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < D / 64; ++i) nk[i] = *reinterpret_cast<const uint4*>(q8 + 64 * i + 16 * quad);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) nv[c] = q8[D + 16 * c + col];
    __builtin_amdgcn_wave_barrier();
}

// The sequence that grid slot b takes when the kernel ranks the lengths itself (no host
// plan): the lengths are ranked longest first (ties by index) and slot b of round
// r = b / R, position pos, takes rank R r + pos in even rounds and R r + (n_r - 1 - pos)
// in odd ones (R = lpt_round, n_r = sequences in that round). Every thread of the
// workgroup calls it; it synchronises the workgroup twice.
template <int W>
__device__ int lpt_pick(const DecodeArgs& a, int b) {
    __shared__ int s_n[kLptMaxSeqs];
    __shared__ int s_pick;
    const int t = threadIdx.x;
    const int max_len = a.max_len;
    for (int i = t; i < a.num_seqs; i += W * 64) {
        const int v = a.seq_lens[i];
        s_n[i] = v < 0 ? 0 : (v > max_len ? max_len : v);
    }
    __syncthreads();
    for (int i = t; i < a.num_seqs; i += W * 64) {
        const int mine = s_n[i];
        int rank = 0;
        for (int k = 0; k < a.num_seqs; ++k) {
            const int o = s_n[k];
            rank += (o > mine) || (o == mine && k < i);
        }
        const int R = a.lpt_round, r = b / R, pos = b - r * R;
        const int hi = min(R, a.num_seqs - r * R);   // sequences in this round
        if (rank == r * R + ((r & 1) ? hi - 1 - pos : pos)) s_pick = i;
    }
    __syncthreads();
    return s_pick;
}

// Merge the per-wave states held in LDS and write out or the partition result.
// sm_m / sm_l: [W][16], sm_o: [W][G][D] (unnormalised accumulators).
template <typename OutT, int D, int W>
__device__ void merge_and_store(const DecodeArgs& a, const float* sm_m, const float* sm_l,
                                const float* sm_o, int b, int g, int p, bool direct) {
    const int G = a.group;
    for (int i = threadIdx.x; i < G * D; i += W * 64) {
        const int h = i / D, dim = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w * 16 + h]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float f = exp2_fast(sm_m[w * 16 + h] - M);  // 0 for a wave with no block
            L += f * sm_l[w * 16 + h];
            O += f * sm_o[(w * G + h) * D + dim];
        }
        const float o = O / L * a.v_scale;
        const int hq = g * G + h;
        if (direct) {
            OutStore<OutT>::st(a.out, (int64_t(b) * a.num_heads + hq) * D + dim, o);
        } else {
            const int64_t row = (int64_t(b) * a.num_heads + hq) * a.max_partitions + p;
            a.part_out[row * D + dim] = o;
            if (dim == 0) {
                a.part_max[row] = M * kLn2;   // back to natural-log units
                a.part_sum[row] = L;
            }
        }
    }
}

// ---------------------------------------------------------------- fp16 / bf16

template <typename T, int D, typename OutT, int W, bool Append, bool F8, int BS, bool PW>
__global__ __launch_bounds__(W * 64) void decode_mfma_kernel(DecodeArgs a) {
    static_assert(D % 64 == 0, "head_dim must be a multiple of 64");
    constexpr int NQK = D / 32;   // 16x16x32 steps for S
    constexpr int NPV = D / 16;   // 16x16x16 steps for O
    constexpr int NKL = F8 ? D / 64 : D / 32;   // 16-byte K loads per tile and lane
    extern __shared__ float lds[];
    float* sm_m = lds;                  // [W][16]
    float* sm_l = lds + W * 16;         // [W][16]
    float* sm_o = lds + 2 * W * 16;     // [W][G][D]

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = a.heads_fastest ? blockIdx.x : blockIdx.y;
    int b = a.heads_fastest ? blockIdx.y : blockIdx.z;
    // PW (fixed partitions): each wave takes a partition of its own, partitions pg W ..
    // pg W + W - 1 of grid slot pg, and writes its record itself. Otherwise the W waves
    // share partition pg and merge through LDS.
    const int pg = a.heads_fastest ? blockIdx.z : blockIdx.x;
    const int p = PW ? pg * W + wave : pg;
    if (a.use_order)
        b = a.order[b];
    else if (a.lpt_round > 0)
        b = lpt_pick<W>(a, b);
    const int G = a.group;
    const int col = lane & 15, quad = lane >> 4;

    // The block ids of this wave's first 64 tiles and the length are read first: memory
    // waits complete in issue order, so loads issued ahead of them (queries, new rows)
    // would hold up the first tile. The context is walked in 16-token tiles (tile j:
    // positions 16j .. 16j + 15), which are blocks for BS = 16, halves of blocks for
    // BS = 32 and pairs of blocks for BS = 8 (tile_ids, load_tile_bs). This wave takes
    // tiles first, first + W, ... of its partition; the table row has max_blocks entries,
    // so the ids are read before the length is known.
    const int blk_begin = p * a.part_tiles;
    constexpr int STEP = PW ? 1 : W;   // tile stride of a wave's list
    const int first = blk_begin + (PW ? 0 : wave);
    const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;
    int tab0, tab0b;
    tile_ids<BS>(table, a.max_blocks, first + lane * STEP, tab0, tab0b);
    const int n_raw = a.seq_lens[b];
    __builtin_amdgcn_sched_barrier(0);

    // Q^T operand (B of the first product): head l%16 of the group, 8 dims per step.
    uint4 qf[NQK];
    {
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + int64_t(b) * a.q_stride +
                               int64_t(g * G + col) * D;
#pragma unroll
        for (int c = 0; c < NQK; ++c)
            qf[c] = col < G ? *reinterpret_cast<const uint4*>(qrow + q_dim<F8>(c, quad))
                            : make_uint4(0, 0, 0, 0);
    }
    // Fused append: the new token's rows, every lane its share in the tile layout: K as
    // the lane's 16-byte K loads hold them (16-bit cache: dims 32c + 8 quad .. + 7; FP8
    // cache: dims 16(4i + quad) .. + 15), V dim 16c + l%16. Kept in registers: reading
    // them from LDS inside the tile loop made the compiler move the tiles to scratch.
    // FP8: each lane loads D/64 consecutive elements of each raw row (nkr, nvr) and, in
    // the wave that stores the row, quantises just those (quantize_new, once its first
    // tiles are on the way); the codes meet in the wave's LDS slice, from which every
    // lane takes the ones it holds in the tile layout (nk, nv). Quantising whole K groups
    // per lane instead cost 40 divisions per lane. Only the wave that stores the row loads
    // it (load_new_rows, once the length has named that wave).
    int slot = -1;
    uint4 nk[Append ? NKL : 1];
    uint32_t nv[Append ? NPV : 1];
    uint32_t nkr = 0, nvr = 0;   // FP8: D/64 raw 16-bit elements each
#pragma unroll
    for (int c = 0; c < (Append ? NKL : 1); ++c) nk[c] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < (Append ? NPV : 1); ++c) nv[c] = 0;
    if constexpr (Append) slot = a.slot_mapping[b];
    auto load_new_rows = [&]() __attribute__((always_inline)) {
        if constexpr (Append) {
            const uint16_t* krow = static_cast<const uint16_t*>(a.new_k) + int64_t(b) * a.new_k_stride +
                                   int64_t(g) * D;
            const uint16_t* vrow = static_cast<const uint16_t*>(a.new_v) + int64_t(b) * a.new_v_stride +
                                   int64_t(g) * D;
            if constexpr (F8) {
                load_new_row_fp8<D>(krow, vrow, lane, nkr, nvr);
            } else {
#pragma unroll
                for (int c = 0; c < NKL; ++c) nk[c] = *reinterpret_cast<const uint4*>(krow + 32 * c + 8 * quad);
#pragma unroll
                for (int c = 0; c < NPV; ++c) nv[c] = vrow[16 * c + col];
            }
        }
    };
    auto quantize_new = [&]() __attribute__((always_inline)) {
        if constexpr (Append && F8)   // in this wave's slice of sm_o, free until the merge
            quantize_new_row_fp8<T, D>(a, reinterpret_cast<uint8_t*>(sm_o + wave * G * D), lane,
                                       nkr, nvr, nk, nv);
    };

    int n = n_raw < 0 ? 0 : (n_raw > a.max_len ? a.max_len : n_raw);
    const int nblk = (n + 15) >> 4;
    const int jl = n > 0 ? (n - 1) >> 4 : -1;     // tile of the newest token
    if ((PW ? pg * W * a.part_tiles : blk_begin) >= nblk) {   // the whole workgroup
        if (pg == 0) write_zero_rows<OutT, D>(a, b, g);
        if constexpr (Append)
            if (pg == 0 && n == 0) write_new_token<T, D, F8, BS>(a, b, g, slot);
        return;
    }
    if (PW && blk_begin >= nblk) return;   // this wave's partition lies past the end
    const int blk_end = min(nblk, blk_begin + a.part_tiles);
    const bool direct = nblk <= a.part_tiles;

    const int nmine = first < blk_end ? (blk_end - first + STEP - 1) / STEP : 0;
    // The wave that holds tile jl (w_new) stores the new rows into the slot. When the
    // slot is the newest position's (what the block pool hands out), w_new overwrites row
    // n-1 of tile jl in its registers with the new token from the key/value inputs once
    // the tile has arrived, so it does not matter whether the store had landed when the
    // tile was read. Otherwise the cache is read as it is. lim: rows below it are valid.
    // (Adding the new token after the last tile as a one-row tile instead cost a whole
    // tile's products on the wave that finishes last.)
    bool subst = false;   // set by w_new when it reaches the table segment holding jl
    const int lim = n;
    const bool own_new = jl >= blk_begin && jl < blk_end;   // this workgroup holds tile jl
    const int w_new = own_new ? (PW ? wave : (jl - blk_begin) % W) : -1;
    const int k_new = own_new ? (jl - first) / STEP : -1;   // jl's index in w_new's list
    if (wave == w_new) load_new_rows();   // wave-uniform
    // The row stores, issued by w_new after its last tile. Stores and loads share one
    // completion counter on this GPU, counted in issue order, so every later tile's wait
    // would include stores issued ahead of its loads; scattered over 128 V rows (one
    // element each) they take microseconds to complete. Issued right after the first tile
    // loads they held up the rest of the wave's stream (8B batch on MI355X: 55.8 us; after
    // the last tile: 53.2 us; with no stores at all: 51.3 us).
    auto store_new_row = [&]() __attribute__((always_inline)) {
        if constexpr (Append) {
            if (wave != w_new) return;
            if (slot < 0 || int64_t(slot) >= a.num_blocks * BS) return;
            const int64_t tile = int64_t(slot / BS) * a.num_kv_heads + g;
            const int off = slot % BS;
            char* kc = const_cast<char*>(static_cast<const char*>(a.k_cache));
            char* vc = const_cast<char*>(static_cast<const char*>(a.v_cache));
            // K ([d/x][BS][x] per block and head): 16-byte group 4c + quad of the row is
            // the lane's nk[c]
            if (col == 0) {
#pragma unroll
                for (int c = 0; c < NKL; ++c)
                    *reinterpret_cast<uint4*>(kc + ((tile * (NKL * 4) + 4 * c + quad) * BS + off) * 16) = nk[c];
            }
            if (quad == 0) {  // V ([d][BS]): dims 16c + col
#pragma unroll
                for (int c = 0; c < NPV; ++c) {
                    if constexpr (F8)
                        reinterpret_cast<uint8_t*>(vc)[(tile * D + 16 * c + col) * BS + off] = uint8_t(nv[c]);
                    else
                        reinterpret_cast<uint16_t*>(vc)[(tile * D + 16 * c + col) * BS + off] = uint16_t(nv[c]);
                }
            }
        }
    };

    f32x4 acc[NPV];
#pragma unroll
    for (int c = 0; c < NPV; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Softmax state per head (lane l: head l%16), in base-2 logit units: m is the
    // reference point of the exponentials, lsum = sum of 2^(x - m) over this lane's
    // tokens. m is the running maximum, except that it is only moved when a block's
    // maximum exceeds it by more than kSlack, so the rescale of acc is rare; every
    // 2^(x - m) stays below 2^kSlack, far from overflow.
    constexpr float kSlack = 8.0f;
    float m = -INFINITY, lsum = 0.f;

    const char* kbase = static_cast<const char*>(a.k_cache);
    const char* vbase = static_cast<const char*>(a.v_cache);
    const int64_t tile_bytes = int64_t(D) * BS * (F8 ? 1 : 2);   // one block of one KV head
    int tab = 0, tabb = 0;   // block ids of the current segment: lane k holds tile k's

    // Issue the loads of tile k of the segment (tile j of the sequence). Returns bit 0
    // set if the id of its (first) block is valid, bit 1 if that of its second block is
    // (BS = 8; always set otherwise). An invalid id breaks the precondition: a safe
    // address is read instead; the tile is skipped (bit 0) or its rows 8-15 masked (bit 1).
    const uint32_t nb_lim = block_limit(a.num_blocks);
    auto load = [&](KvTile<D, F8>& t, int k, int j) -> int {
        const int ida = __builtin_amdgcn_readlane(tab, k);
        const bool oka = uint32_t(ida) < nb_lim;
        const int64_t pa = oka ? ida : 0;
        int64_t pb = pa;
        bool okb = true;
        if constexpr (BS == 8) {
            const int idb = __builtin_amdgcn_readlane(tabb, k);
            okb = uint32_t(idb) < nb_lim;
            pb = okb ? idb : 0;
        }
        const int64_t ta = pa * a.num_kv_heads + g, tb = pb * a.num_kv_heads + g;
        load_tile_bs<D, BS>(t, kbase + ta * tile_bytes, vbase + ta * tile_bytes,
                            kbase + tb * tile_bytes, vbase + tb * tile_bytes, 16 * (j & 1), lane);
        return int(oka) | (int(okb) << 1);
    };

    // A tile whose block id broke the precondition (ok bit 0 clear) was read from block 0
    // and is masked out entirely by arithmetic, not skipped by a branch: every loaded
    // register is then consumed on every path, so the compiler's memory waits stay per
    // tile (a path that skips a tile's registers makes it drain all outstanding loads at
    // the loop head). An invalid second block (BS = 8) masks rows 8-15.
    auto compute = [&](KvTile<D, F8>& t, int j, int ok) __attribute__((always_inline)) {
        if constexpr (Append) {
            if (subst && j == jl) {   // wave-uniform: row n-1 of tile jl is the new token
                // bit masks, not selects between the arrays: a select of two loads would
                // put the tile and the row in scratch memory to load through a pointer
                const int off = (n - 1) & 15;
                const bool vl = quad == (off >> 2);
                const uint32_t km = col == off ? 0xffffffffu : 0u;
#pragma unroll
                for (int c = 0; c < NKL; ++c) {
                    t.k[c].x = (t.k[c].x & ~km) | (nk[c].x & km);
                    t.k[c].y = (t.k[c].y & ~km) | (nk[c].y & km);
                    t.k[c].z = (t.k[c].z & ~km) | (nk[c].z & km);
                    t.k[c].w = (t.k[c].w & ~km) | (nk[c].w & km);
                }
                const int e = off & 3;   // the row's element in the lane's V word(s)
                if constexpr (F8) {
                    const uint32_t sh = 8u * uint32_t(e), mk = vl ? 0xffu << sh : 0u;
#pragma unroll
                    for (int c = 0; c < NPV; ++c) t.v[c] = (t.v[c] & ~mk) | (((nv[c] & 0xffu) << sh) & mk);
                } else {
                    const uint32_t sh = 16u * uint32_t(e & 1);
                    const uint32_t mx = vl && e < 2 ? 0xffffu << sh : 0u;
                    const uint32_t my = vl && e >= 2 ? 0xffffu << sh : 0u;
#pragma unroll
                    for (int c = 0; c < NPV; ++c) {
                        const uint32_t r = (nv[c] & 0xffffu) << sh;
                        t.v[c].x = (t.v[c].x & ~mx) | (r & mx);
                        t.v[c].y = (t.v[c].y & ~my) | (r & my);
                    }
                }
            }
        }
        const int lim_t = !(ok & 1) ? j * 16 : (ok & 2) ? lim : min(lim, j * 16 + 8);
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NQK; ++c) s = Mfma<T>::qk(k_operand<T, D>(t, c), qf[c], s);

        const int tok0 = j * 16 + 4 * quad;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = tok0 + e < lim_t ? s[e] * a.scale_log2 : -INFINITY;
        const float bm = max_over_rows(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const bool move = bm > m + kSlack;          // true on the first block (m = -inf)
        if (__builtin_amdgcn_ballot_w64(move)) {    // wave-uniform, rare after the first block
            const float mn = move ? bm : m;
            const float alpha = exp2_fast(m - mn);   // 1 where m stays, 0 from -inf
            lsum *= alpha;
#pragma unroll
            for (int c = 0; c < NPV; ++c) acc[c] *= alpha;
            m = mn;
        }
        float pe[4];   // a masked row gives 0, also while m is still -inf
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = x[e] == -INFINITY ? 0.f : exp2_fast(x[e] - m);
        lsum += (pe[0] + pe[1]) + (pe[2] + pe[3]);

        if (j * 16 + 16 > lim_t)   // partly filled tile: rows from lim_t on may hold anything
            mask_rows<D>(t, tok0 + 0 < lim_t, tok0 + 1 < lim_t, tok0 + 2 < lim_t, tok0 + 3 < lim_t);
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) Mfma<T>::split(pe[e], hi[e], lo[e]);
        const uint2 phi = make_uint2(uint32_t(hi[0]) | (uint32_t(hi[1]) << 16),
                                     uint32_t(hi[2]) | (uint32_t(hi[3]) << 16));
        const uint2 plo = make_uint2(uint32_t(lo[0]) | (uint32_t(lo[1]) << 16),
                                     uint32_t(lo[2]) | (uint32_t(lo[3]) << 16));
#pragma unroll
        for (int c = 0; c < NPV; ++c) {
            const uint2 vv = v_operand<T, D>(t, c);
            acc[c] = Mfma<T>::pv(vv, phi, acc[c]);
            acc[c] = Mfma<T>::pv(vv, plo, acc[c]);
        }
    };

    // Segments of up to 64 blocks (one block id per lane). Inside a segment a wave keeps NB
    // tiles in flight: the loads of tile k + NB - 1 are issued before tile k is used, so
    // NB - 1 loads stay outstanding while a tile is computed and the wait for the current
    // tile never waits for a later one. Past the end of the segment the loads repeat its
    // last tile (no data-dependent branch around them). Tiles of one stage each, also for
    // the half-size FP8 tiles (stages of two measured slower).
    constexpr int NB = kDecodeBuffers;
    static_assert(NB >= 1 && NB <= 3, "one to three tiles in flight");
    for (int k0 = 0; k0 < nmine; k0 += 64) {
        const int cnt = min(64, nmine - k0);
        if (k0 == 0) {
            tab = tab0;
            tabb = tab0b;
        } else {
            tile_ids<BS>(table, a.max_blocks, lane < cnt ? first + (k0 + lane) * STEP : a.max_tiles,
                         tab, tabb);
        }
        if constexpr (Append) {
            if (wave == w_new && k_new >= k0 && k_new < k0 + 64) {   // wave-uniform
                // the block holding position n - 1: tile jl's, or for BS = 8 its first or
                // second block
                const int half = BS == 8 && ((n - 1) & 15) >= 8;
                const int64_t phys_l = __builtin_amdgcn_readlane(half ? tabb : tab, k_new - k0);
                subst = slot >= 0 && phys_l >= 0 && phys_l < a.num_blocks &&
                        int64_t(slot) == phys_l * BS + (n - 1) % BS;
            }
        }
        KvTile<D, F8> X, Y, Z;
        int okX = 0, okY = 0, okZ = 0;
        auto tile_of = [&](int k) { return first + (k0 + k) * STEP; };
        // The scheduling barrier keeps each tile's loads issued before the previous tile's
        // arithmetic: left free, the compiler hoists that arithmetic (and its wait) above
        // them, so the next tile is requested only after the current one has arrived.
        auto ld = [&](KvTile<D, F8>& t, int k) {
            const int kk = min(k, cnt - 1);
            const int ok = load(t, kk, tile_of(kk));
            __builtin_amdgcn_sched_barrier(0);
            return ok;
        };
        okX = ld(X, 0);
        if constexpr (NB == 3) okY = ld(Y, 1);
        if (k0 == 0 && wave == w_new) quantize_new();   // FP8: the codes, for tile jl too
        if constexpr (NB == 1) {
            for (int k = 0; k < cnt; ++k) {
                if (k > 0) okX = ld(X, k);
                compute(X, tile_of(k), okX);
            }
        } else if constexpr (NB == 2) {
            for (int k = 0; k < cnt; k += 2) {
                okY = ld(Y, k + 1);
                compute(X, tile_of(k), okX);
                if (k + 1 >= cnt) break;
                okX = ld(X, k + 2);
                compute(Y, tile_of(k + 1), okY);
            }
        } else {
            for (int k = 0; k < cnt; k += 3) {
                okZ = ld(Z, k + 2);
                compute(X, tile_of(k), okX);
                if (k + 1 >= cnt) break;
                okX = ld(X, k + 3);
                compute(Y, tile_of(k + 1), okY);
                if (k + 2 >= cnt) break;
                okY = ld(Y, k + 4);
                compute(Z, tile_of(k + 2), okZ);
            }
        }
    }

    store_new_row();

    // lanes l, l^16, l^32, l^48 hold the same head: total its running sum
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);

    if constexpr (PW) {   // this wave's partition alone: its result as merge_and_store forms it
        if (col < G) {
            const int hq = g * G + col;
            if (direct) {
#pragma unroll
                for (int c = 0; c < NPV; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        OutStore<OutT>::st(a.out, (int64_t(b) * a.num_heads + hq) * D + 16 * c + 4 * quad + e,
                                           acc[c][e] / lsum * a.v_scale);
            } else {
                const int64_t row = (int64_t(b) * a.num_heads + hq) * a.max_partitions + p;
#pragma unroll
                for (int c = 0; c < NPV; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        a.part_out[row * D + 16 * c + 4 * quad + e] = acc[c][e] / lsum * a.v_scale;
                if (quad == 0) {
                    a.part_max[row] = m * kLn2;   // back to natural-log units
                    a.part_sum[row] = lsum;
                }
            }
        }
        return;
    }
    if (lane < 16) {
        sm_m[wave * 16 + lane] = m;
        sm_l[wave * 16 + lane] = lsum;
    }
    if (col < G) {
#pragma unroll
        for (int c = 0; c < NPV; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) sm_o[(wave * G + col) * D + 16 * c + 4 * quad + e] = acc[c][e];
    }
    __syncthreads();
    merge_and_store<OutT, D, W>(a, sm_m, sm_l, sm_o, b, g, p, direct);
}

// ------------------------------------------------ 32-token blocks, whole blocks
// Caches at 32 tokens per block (FP8 and 16-bit), single pass or partitions of whole
// blocks. The 16-token tiles of decode_mfma_kernel read half of every V row there (32 of
// 64 bytes at 16 bits, 16 of 32 at FP8), so each V load instruction touches twice the
// sectors of the 16-token case and the other half is fetched again by another wave. Here
// a wave takes whole blocks: the two QK products of a block read their K rows in a
// permuted order (MFMA row r of product A: position 8 (r / 4) + r % 4 of the block, of
// product B that + 4), so lane l holds the logits of positions 8 (l/16) .. + 7, which are
// its 8 k-slots of one 16x16x32 PV product in both operands. Its V operand is then one
// load of those 8 positions of a dimension row (8 bytes of codes, or 16 bytes at 16 bits):
// the block's V rows are read whole, with half the load instructions.
// Softmax, reference points, merging and the fused append are those of decode_mfma_kernel.
template <int D, bool F8> struct KvBlock32;
template <int D> struct KvBlock32<D, true> {
    uint4 ka[D / 64];   // K rows of product A: 16 codes (dims 16 (4 i + quad) ..) each
    uint4 kb[D / 64];   // product B
    uint2 v[D / 16];    // positions 8 quad .. + 7 of dimension 16 c + col
};
template <int D> struct KvBlock32<D, false> {
    uint4 ka[D / 32];   // K rows of product A: dims 32 c + 8 quad .. + 7 (QK step c)
    uint4 kb[D / 32];   // product B
    uint4 v[D / 16];    // positions 8 quad .. + 7 of dimension 16 c + col
};

// A wave keeps one block in flight (16 KiB at 16 bits, 8 KiB of codes). On MI355X, 8B
// batch at 32 tokens per block: bf16 55.6 us per launch against 59.1 with two blocks per
// wave (64 MiB in flight over the chip; a gather of the 16-token tiles is fastest at 16-32
// MiB), FP8 30.2 against 31.4-32.3.
template <typename T, int D, typename OutT, int W, bool Append, bool F8>
__global__ __launch_bounds__(W * 64) void decode_blk32_kernel(DecodeArgs a) {
    static_assert(D % 64 == 0, "head_dim must be a multiple of 64");
    constexpr int BS = 32;
    constexpr int NQK = D / 32;   // 16x16x32 steps for S
    constexpr int NPV = D / 16;   // 16x16x32 steps for O (32 positions each)
    constexpr int NKL = F8 ? D / 64 : D / 32;   // 16-byte K loads per product and lane
    extern __shared__ float lds[];
    float* sm_m = lds;                  // [W][16]
    float* sm_l = lds + W * 16;         // [W][16]
    float* sm_o = lds + 2 * W * 16;     // [W][G][D]

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = a.heads_fastest ? blockIdx.x : blockIdx.y;
    int b = a.heads_fastest ? blockIdx.y : blockIdx.z;
    const int p = a.heads_fastest ? blockIdx.z : blockIdx.x;
    if (a.use_order)
        b = a.order[b];
    else if (a.lpt_round > 0)
        b = lpt_pick<W>(a, b);
    const int G = a.group;
    const int col = lane & 15, quad = lane >> 4;
    const int ra = 8 * (col >> 2) + (col & 3), rb = ra + 4;   // this lane's K rows of A, B

    // block ids and length first (see decode_mfma_kernel); this wave takes blocks first,
    // first + W, ... of its partition
    const int part_blocks = a.part_tiles >> 1;
    const int blk_begin = p * part_blocks;
    const int first = blk_begin + wave;
    const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;
    const int tab0 = first + lane * W < a.max_blocks ? table[first + lane * W] : -1;
    const int n_raw = a.seq_lens[b];
    __builtin_amdgcn_sched_barrier(0);

    uint4 qf[NQK];
    {
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + int64_t(b) * a.q_stride +
                               int64_t(g * G + col) * D;
#pragma unroll
        for (int c = 0; c < NQK; ++c)
            qf[c] = col < G ? *reinterpret_cast<const uint4*>(qrow + q_dim<F8>(c, quad))
                            : make_uint4(0, 0, 0, 0);
    }
    // fused append: every lane loads D/64 consecutive raw elements of the new K and V rows
    // (nkr, nvr). FP8: the wave that stores the row quantises them, and every lane keeps
    // the codes it holds in the tile layout (nk: K group 4c + quad; nv: dimension 16c +
    // col). 16-bit: that wave puts the row into its slice of sm_o (free until the merge;
    // K at elements [0, D), V at [D, 2D)), read only where the row is substituted or
    // stored: held in registers through the loop it pushed the two blocks in flight into
    // scratch.
    int slot = -1;
    constexpr bool kRegRow = Append && F8;
    uint4 nk[kRegRow ? NKL : 1];
    uint32_t nv[kRegRow ? NPV : 1];
    uint32_t nkr = 0, nvr = 0;
    uint16_t* nrow = reinterpret_cast<uint16_t*>(sm_o + wave * G * D);
    if constexpr (Append) {
        slot = a.slot_mapping[b];
        const uint16_t* krow = static_cast<const uint16_t*>(a.new_k) + int64_t(b) * a.new_k_stride +
                               int64_t(g) * D;
        const uint16_t* vrow = static_cast<const uint16_t*>(a.new_v) + int64_t(b) * a.new_v_stride +
                               int64_t(g) * D;
        load_new_row_fp8<D>(krow, vrow, lane, nkr, nvr);
    }
    auto quantize_new = [&]() __attribute__((always_inline)) {
        if constexpr (Append && F8) {
            quantize_new_row_fp8<T, D>(a, reinterpret_cast<uint8_t*>(sm_o + wave * G * D), lane,
                                       nkr, nvr, nk, nv);
        } else if constexpr (Append) {
            if constexpr (D == 128) {
                *reinterpret_cast<uint32_t*>(nrow + 2 * lane) = nkr;
                *reinterpret_cast<uint32_t*>(nrow + D + 2 * lane) = nvr;
            } else {
                nrow[lane] = uint16_t(nkr);
                nrow[D + lane] = uint16_t(nvr);
            }
            __builtin_amdgcn_wave_barrier();
        }
    };
    auto new_k = [&](int c) __attribute__((always_inline)) -> uint4 {   // K group 4c + quad
        if constexpr (kRegRow) return nk[c];
        else return *reinterpret_cast<const uint4*>(nrow + 32 * c + 8 * quad);
    };
    auto new_v = [&](int c) __attribute__((always_inline)) -> uint32_t {   // dimension 16c + col
        if constexpr (kRegRow) return nv[c];
        else return nrow[D + 16 * c + col];
    };

    int n = n_raw < 0 ? 0 : (n_raw > a.max_len ? a.max_len : n_raw);
    const int nblk = (n + BS - 1) / BS;
    const int jl = n > 0 ? (n - 1) / BS : -1;    // block of the newest token
    if (blk_begin >= nblk) {
        if (p == 0) write_zero_rows<OutT, D>(a, b, g);
        if constexpr (Append)
            if (p == 0 && n == 0) write_new_token<T, D, F8, BS>(a, b, g, slot);
        return;
    }
    const int blk_end = min(nblk, blk_begin + part_blocks);
    const bool direct = nblk <= part_blocks;
    const int nmine = first < blk_end ? (blk_end - first + W - 1) / W : 0;
    // w_new puts the new token into row n-1 of block jl in its registers (as
    // decode_mfma_kernel does for its tiles)
    bool subst = false;
    const int lim = n;
    const bool own_new = jl >= blk_begin && jl < blk_end;
    const int w_new = own_new ? (jl - blk_begin) % W : -1;
    const int k_new = own_new ? (jl - first) / W : -1;
    // the row stores, by w_new after its last block (see decode_mfma_kernel)
    auto store_new_row = [&]() __attribute__((always_inline)) {
        if constexpr (Append) {
            if (wave != w_new) return;
            if (slot < 0 || int64_t(slot) >= a.num_blocks * BS) return;
            const int64_t tile = int64_t(slot / BS) * a.num_kv_heads + g;
            const int off = slot % BS;
            char* kc = const_cast<char*>(static_cast<const char*>(a.k_cache));
            char* vc = const_cast<char*>(static_cast<const char*>(a.v_cache));
            if (col == 0) {
#pragma unroll
                for (int c = 0; c < NKL; ++c)
                    *reinterpret_cast<uint4*>(kc + ((tile * (NKL * 4) + 4 * c + quad) * BS + off) * 16) = new_k(c);
            }
            if (quad == 0) {
#pragma unroll
                for (int c = 0; c < NPV; ++c) {
                    if constexpr (F8)
                        reinterpret_cast<uint8_t*>(vc)[(tile * D + 16 * c + col) * BS + off] = uint8_t(new_v(c));
                    else
                        reinterpret_cast<uint16_t*>(vc)[(tile * D + 16 * c + col) * BS + off] = uint16_t(new_v(c));
                }
            }
        }
    };

    f32x4 acc[NPV];
#pragma unroll
    for (int c = 0; c < NPV; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr float kSlack = 8.0f;
    float m = -INFINITY, lsum = 0.f;

    const char* kbase = static_cast<const char*>(a.k_cache);
    const char* vbase = static_cast<const char*>(a.v_cache);
    constexpr int64_t tile_bytes = int64_t(D) * BS * (F8 ? 1 : 2);   // one block of one KV head
    int tab = 0;

    // Issue the loads of segment block k; false if its id is invalid (a safe address is
    // read and the block is skipped).
    const uint32_t nb_lim = block_limit(a.num_blocks);
    auto load = [&](KvBlock32<D, F8>& t, int k) -> bool {
        const int id = __builtin_amdgcn_readlane(tab, k);
        const bool ok = uint32_t(id) < nb_lim;
        const int64_t pa = ok ? id : 0;
        const buf_rsrc_t kr = tile_rsrc(kbase + (pa * a.num_kv_heads + g) * tile_bytes, int(tile_bytes));
        const buf_rsrc_t vr = tile_rsrc(vbase + (pa * a.num_kv_heads + g) * tile_bytes, int(tile_bytes));
#pragma unroll
        for (int i = 0; i < NKL; ++i) {   // K group 4 i + quad of rows ra, rb
            t.ka[i] = bld16(kr, ((4 * i + quad) * BS + ra) * 16);
            t.kb[i] = bld16(kr, ((4 * i + quad) * BS + rb) * 16);
        }
#pragma unroll
        for (int c = 0; c < NPV; ++c) {
            if constexpr (F8)
                t.v[c] = bld8(vr, (16 * c + col) * BS + 8 * quad);
            else
                t.v[c] = bld16(vr, ((16 * c + col) * BS + 8 * quad) * 2);
        }
        return ok;
    };
    // the K operand of QK step c from the loaded groups (FP8: 8 of 16 codes, widened)
    auto kop = [](const uint4* w, int c) {
        if constexpr (F8) {
            const uint4 q = w[c >> 1];
            const uint2 lo = Fp8<T>::x4((c & 1) ? q.z : q.x), hi = Fp8<T>::x4((c & 1) ? q.w : q.y);
            return make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
            return w[c];
        }
    };

    // block jb (positions 32 jb .. + 31); positions below lim are valid. An invalid block
    // id (read from block 0) is masked out by arithmetic, not skipped (see decode_mfma_kernel).
    auto compute = [&](KvBlock32<D, F8>& t, int jb, bool ok) __attribute__((always_inline)) {
        if constexpr (Append) {
            if (subst && jb == jl) {   // wave-uniform: position off of block jl is the new token
                // MFMA row r of product A holds position 8 (r / 4) + r % 4, of product B that
                // + 4; in the lanes with quad == off / 8, V word h holds positions 8 quad +
                // 4 h .. + 3 (codes) or 8 quad + 2 h, + 1 (16-bit). Bit masks, not selects
                // between arrays (see decode_mfma_kernel).
                const int off = (n - 1) % BS;
                const int r = 4 * (off >> 3) + (off & 3);
                const bool inb = (off & 7) >= 4;
                const uint32_t ma = col == r && !inb ? 0xffffffffu : 0u;
                const uint32_t mb = col == r && inb ? 0xffffffffu : 0u;
#pragma unroll
                for (int c = 0; c < NKL; ++c) {
                    const uint4 w = new_k(c);
                    t.ka[c].x = (t.ka[c].x & ~ma) | (w.x & ma);
                    t.ka[c].y = (t.ka[c].y & ~ma) | (w.y & ma);
                    t.ka[c].z = (t.ka[c].z & ~ma) | (w.z & ma);
                    t.ka[c].w = (t.ka[c].w & ~ma) | (w.w & ma);
                    t.kb[c].x = (t.kb[c].x & ~mb) | (w.x & mb);
                    t.kb[c].y = (t.kb[c].y & ~mb) | (w.y & mb);
                    t.kb[c].z = (t.kb[c].z & ~mb) | (w.z & mb);
                    t.kb[c].w = (t.kb[c].w & ~mb) | (w.w & mb);
                }
                const bool vq = quad == (off >> 3);
                if constexpr (F8) {
                    const uint32_t sh = 8u * uint32_t(off & 3);
                    const uint32_t mx = vq && !inb ? 0xffu << sh : 0u;
                    const uint32_t my = vq && inb ? 0xffu << sh : 0u;
#pragma unroll
                    for (int c = 0; c < NPV; ++c) {
                        const uint32_t code = (new_v(c) & 0xffu) << sh;
                        t.v[c].x = (t.v[c].x & ~mx) | (code & mx);
                        t.v[c].y = (t.v[c].y & ~my) | (code & my);
                    }
                } else {
                    const uint32_t sh = 16u * uint32_t(off & 1);
                    const int h = (off & 7) >> 1;
                    const uint32_t mw = 0xffffu << sh;
                    const uint32_t m0 = vq && h == 0 ? mw : 0u, m1 = vq && h == 1 ? mw : 0u;
                    const uint32_t m2 = vq && h == 2 ? mw : 0u, m3 = vq && h == 3 ? mw : 0u;
#pragma unroll
                    for (int c = 0; c < NPV; ++c) {
                        const uint32_t e = (new_v(c) & 0xffffu) << sh;
                        t.v[c].x = (t.v[c].x & ~m0) | (e & m0);
                        t.v[c].y = (t.v[c].y & ~m1) | (e & m1);
                        t.v[c].z = (t.v[c].z & ~m2) | (e & m2);
                        t.v[c].w = (t.v[c].w & ~m3) | (e & m3);
                    }
                }
            }
        }
        const int lim_b = ok ? lim : jb * BS;
        const int p0 = jb * BS + 8 * quad;   // this lane's 8 positions
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NQK; ++c) {
            sa = Mfma<T>::qk(kop(t.ka, c), qf[c], sa);
            sb = Mfma<T>::qk(kop(t.kb, c), qf[c], sb);
        }
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = p0 + e < lim_b ? sa[e] * a.scale_log2 : -INFINITY;
            x[4 + e] = p0 + 4 + e < lim_b ? sb[e] * a.scale_log2 : -INFINITY;
        }
        const float bm = max_over_rows(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                             fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
        const bool move = bm > m + kSlack;
        if (__builtin_amdgcn_ballot_w64(move)) {
            const float mn = move ? bm : m;
            const float alpha = exp2_fast(m - mn);
            lsum *= alpha;
#pragma unroll
            for (int c = 0; c < NPV; ++c) acc[c] *= alpha;
            m = mn;
        }
        const float mref = m == -INFINITY ? 0.f : m;
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = exp2_fast(x[e] - mref);
        lsum += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
        if (jb * BS + BS > lim_b) {   // partly valid block: rows from lim_b on may hold anything
            if constexpr (F8) {
                uint32_t m0 = 0, m1 = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    m0 |= (p0 + e < lim_b ? 0xffu : 0u) << (8 * e);
                    m1 |= (p0 + 4 + e < lim_b ? 0xffu : 0u) << (8 * e);
                }
#pragma unroll
                for (int c = 0; c < NPV; ++c) {
                    t.v[c].x &= m0;
                    t.v[c].y &= m1;
                }
            } else {
                uint32_t mw[4];
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    mw[h] = (p0 + 2 * h < lim_b ? 0xffffu : 0u) | (p0 + 2 * h + 1 < lim_b ? 0xffff0000u : 0u);
#pragma unroll
                for (int c = 0; c < NPV; ++c) {
                    t.v[c].x &= mw[0];
                    t.v[c].y &= mw[1];
                    t.v[c].z &= mw[2];
                    t.v[c].w &= mw[3];
                }
            }
        }
        uint16_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) Mfma<T>::split(pe[e], hi[e], lo[e]);
        const uint4 phi = make_uint4(uint32_t(hi[0]) | (uint32_t(hi[1]) << 16),
                                     uint32_t(hi[2]) | (uint32_t(hi[3]) << 16),
                                     uint32_t(hi[4]) | (uint32_t(hi[5]) << 16),
                                     uint32_t(hi[6]) | (uint32_t(hi[7]) << 16));
        const uint4 plo = make_uint4(uint32_t(lo[0]) | (uint32_t(lo[1]) << 16),
                                     uint32_t(lo[2]) | (uint32_t(lo[3]) << 16),
                                     uint32_t(lo[4]) | (uint32_t(lo[5]) << 16),
                                     uint32_t(lo[6]) | (uint32_t(lo[7]) << 16));
#pragma unroll
        for (int c = 0; c < NPV; ++c) {
            uint4 vv;
            if constexpr (F8) {
                const uint2 w0 = Fp8<T>::x4(t.v[c].x), w1 = Fp8<T>::x4(t.v[c].y);
                vv = make_uint4(w0.x, w0.y, w1.x, w1.y);
            } else {
                vv = t.v[c];
            }
            acc[c] = Mfma<T>::qk(vv, phi, acc[c]);
            acc[c] = Mfma<T>::qk(vv, plo, acc[c]);
        }
    };

    // segments of up to 64 blocks (one block id per lane), two blocks in flight
    for (int k0 = 0; k0 < nmine; k0 += 64) {
        const int cnt = min(64, nmine - k0);
        if (k0 == 0) {
            tab = tab0;
        } else {
            const int jb = first + (k0 + lane) * W;
            tab = lane < cnt && jb < a.max_blocks ? table[jb] : -1;
        }
        if constexpr (Append) {
            if (wave == w_new && k_new >= k0 && k_new < k0 + 64) {   // wave-uniform
                const int64_t phys_l = __builtin_amdgcn_readlane(tab, k_new - k0);
                subst = slot >= 0 && phys_l >= 0 && phys_l < a.num_blocks &&
                        int64_t(slot) == phys_l * BS + (n - 1) % BS;
            }
        }
        auto blk_of = [&](int k) { return first + (k0 + k) * W; };
        KvBlock32<D, F8> X;   // one block in flight
        bool okX = load(X, 0);
        if (k0 == 0 && wave == w_new) quantize_new();   // the new row, for block jl too
        for (int k = 0; k < cnt; ++k) {
            if (k > 0) okX = load(X, k);
            compute(X, blk_of(k), okX);
        }
    }

    store_new_row();

    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (lane < 16) {
        sm_m[wave * 16 + lane] = m;
        sm_l[wave * 16 + lane] = lsum;
    }
    if (col < G) {
#pragma unroll
        for (int c = 0; c < NPV; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) sm_o[(wave * G + col) * D + 16 * c + 4 * quad + e] = acc[c][e];
    }
    __syncthreads();
    merge_and_store<OutT, D, W>(a, sm_m, sm_l, sm_o, b, g, p, direct);
}

// ------------------------------------------------------- fp16 / bf16, balanced split
// Same per-tile arithmetic as decode_mfma_kernel; the work is cut as described in
// split.hpp. Each wave is independent: it reads the block ids of up to 64 of its tiles
// with one vector load (lane k: tile k), then streams the tiles, switching (sequence,
// KV head) at piece boundaries. A piece covering all of its (b, g) is written to out;
// any other piece becomes an (o, m, l) record at piece index u - floor(start / s).
//
// Finished pieces are parked in LDS result slots of the wave and written to HBM only
// after its last tile (or when the slots are full). On gfx950 one counter tracks both
// outstanding loads and outstanding stores, so a store issued between tile loads makes
// every later tile wait for the store's completion as well; parking the results keeps
// the stream of tile loads free of stores.
constexpr int kSplitPiecesPerBatch = 4;   // queries staged in LDS per wave and batch
constexpr int kSplitStage = 1;            // tiles per pipeline stage
constexpr int kSplitMaxSlots = 8;         // result slots per wave (upper bound)
constexpr int kSplitWaveLds = 17920;      // LDS bytes per wave: staged queries + slots

// Per-wave LDS of the balanced split: staged queries, then `slots` result slots of
// (G*D outputs, G reference points, G sums) floats, then 4 ints of metadata per slot.
__host__ __device__ constexpr int split_q_bytes(int G, int D) { return kSplitPiecesPerBatch * G * D * 2; }
__host__ __device__ constexpr int split_slot_floats(int G, int D) { return (G * D + 2 * G + 3) & ~3; }
__host__ __device__ constexpr int split_wave_bytes(int G, int D, int slots) {
    return split_q_bytes(G, D) + slots * (split_slot_floats(G, D) * 4 + 16);
}

template <typename T, int D, typename OutT, bool F8, int BS>
__global__ __launch_bounds__(kSplitThreads) void decode_split_kernel(DecodeArgs a) {
    constexpr int NQK = D / 32, NPV = D / 16;
    constexpr int kWaves = kSplitThreads / 64;
    __shared__ int32_t s_end[kSplitMaxSeqs];
    __shared__ int32_t s_len[kSplitMaxSeqs];
    __shared__ int32_t s_wave[kWaves];
    extern __shared__ uint4 s_dyn[];    // per wave: see split_wave_bytes
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int col = lane & 15, quad = lane >> 4;
    const int G = a.group, hkv = a.num_kv_heads;
    const int total = split_scan(a.seq_lens, a.num_seqs, hkv, a.max_len, s_end, s_len, s_wave);
    const int share = split_share(total, a.split);
    const int u = blockIdx.x * kWaves + wave;
    const int64_t t0l = int64_t(u) * share;
    if (t0l >= total) return;
    const int t0 = int(t0l);
    const int t1 = min(total, t0 + share);

    const char* kbase = static_cast<const char*>(a.k_cache);
    const char* vbase = static_cast<const char*>(a.v_cache);
    const int64_t tile_bytes = int64_t(D) * BS * (F8 ? 1 : 2);   // one block of one KV head
    const int qpiece = G * D;                              // elements per staged query set
    char* my_lds = reinterpret_cast<char*>(s_dyn) + wave * split_wave_bytes(G, D, a.slots);
    uint16_t* my_q = reinterpret_cast<uint16_t*>(my_lds);
    const int slot_floats = split_slot_floats(G, D);
    float* slots = reinterpret_cast<float*>(my_lds + split_q_bytes(G, D));
    int32_t* slot_meta = reinterpret_cast<int32_t*>(slots + a.slots * slot_floats);
    int nused = 0;   // result slots in use (wave-uniform)
    constexpr float kSlack = 8.0f;

    // state of the current piece
    uint4 qf[NQK];
    f32x4 acc[NPV];
    float m = -INFINITY, lsum = 0.f;
    int cur_bg = -1, seg_b = 0, seg_g = 0, seg_n = 0, seg_nblk = 0, seg_start = 0;
    int first_j = 0, last_j = 0, piece_slot = -1;

    auto begin_piece = [&](int bg, int j) {
        seg_b = bg / hkv;
        seg_g = bg - seg_b * hkv;
        seg_n = s_len[seg_b];
        seg_nblk = (seg_n + 15) >> 4;
        seg_start = (seg_b ? s_end[seg_b - 1] : 0) + seg_g * seg_nblk;
        first_j = j;
        cur_bg = bg;
        ++piece_slot;
        const uint16_t* qs = my_q + piece_slot * qpiece + (col < G ? col : 0) * D;
#pragma unroll
        for (int c = 0; c < NQK; ++c)
            qf[c] = col < G ? *reinterpret_cast<const uint4*>(qs + q_dim<F8>(c, quad))
                            : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < NPV; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        lsum = 0.f;
    };

    // Write the parked results: G*D outputs per slot, four consecutive ones per lane
    // and store (the G heads of a group are consecutive rows of out).
    auto flush = [&]() {
        __builtin_amdgcn_wave_barrier();
        for (int sl = 0; sl < nused; ++sl) {
            const float* so = slots + sl * slot_floats;
            const int b = slot_meta[4 * sl], g = slot_meta[4 * sl + 1], piece = slot_meta[4 * sl + 2];
            const int64_t head0 = int64_t(b) * a.num_heads + g * G;
            for (int i = 4 * lane; i < G * D; i += 256) {
                const float4 v = *reinterpret_cast<const float4*>(so + i);
                if (piece < 0) {
                    OutStore<OutT>::st4(a.out, head0 * D + i, v);
                } else {
                    const int64_t row = (head0 + i / D) * a.max_partitions + piece;
                    *reinterpret_cast<float4*>(a.part_out + row * D + i % D) = v;
                }
            }
            if (piece >= 0 && lane < G) {
                const int64_t row = (head0 + lane) * a.max_partitions + piece;
                a.part_max[row] = so[G * D + lane];
                a.part_sum[row] = so[G * D + G + lane];
            }
        }
        nused = 0;
        __builtin_amdgcn_wave_barrier();
    };

    // Park the finished piece in the next result slot (normalised outputs; the
    // reference point in natural-log units and the sum for the reduce).
    auto end_piece = [&]() {
        float L = lsum;
        L += __shfl_xor(L, 16, 64);
        L += __shfl_xor(L, 32, 64);
        if (nused == a.slots) flush();
        float* so = slots + nused * slot_floats;
        if (col < G) {
            const float inv = a.v_scale / L;
#pragma unroll
            for (int c = 0; c < NPV; ++c)
                *reinterpret_cast<float4*>(so + col * D + 16 * c + 4 * quad) =
                    make_float4(acc[c][0] * inv, acc[c][1] * inv, acc[c][2] * inv, acc[c][3] * inv);
            if (quad == 0) {
                so[G * D + col] = m * kLn2;
                so[G * D + G + col] = L;
            }
        }
        if (lane == 0) {
            const bool whole = first_j == 0 && last_j == seg_nblk - 1;
            slot_meta[4 * nused] = seg_b;
            slot_meta[4 * nused + 1] = seg_g;
            slot_meta[4 * nused + 2] = whole ? -1 : u - seg_start / share;
        }
        ++nused;
    };

    // per-lane metadata of the current batch: tile k's block ids (tphys; tphysb the
    // second block for BS = 8), (b, g) and tile index j
    int tphys = 0, tphysb = 0, tbg = 0, tj = 0;
    const uint32_t nb_lim = block_limit(a.num_blocks);
    // bit 0: the (first) block id is valid; bit 1: the second one (BS = 8) is
    auto load = [&](KvTile<D, F8>& t, int k) -> int {
        const int ida = __builtin_amdgcn_readlane(tphys, k);
        const bool oka = uint32_t(ida) < nb_lim;
        const int64_t pa = oka ? ida : 0;
        int64_t pb = pa;
        bool okb = true;
        if constexpr (BS == 8) {
            const int idb = __builtin_amdgcn_readlane(tphysb, k);
            okb = uint32_t(idb) < nb_lim;
            pb = okb ? idb : 0;
        }
        const int g = __builtin_amdgcn_readlane(tbg, k) % hkv;
        const int j = __builtin_amdgcn_readlane(tj, k);
        const int64_t ta = pa * hkv + g, tb = pb * hkv + g;
        load_tile_bs<D, BS>(t, kbase + ta * tile_bytes, vbase + ta * tile_bytes,
                            kbase + tb * tile_bytes, vbase + tb * tile_bytes, 16 * (j & 1), lane);
        return int(oka) | (int(okb) << 1);
    };

    auto compute = [&](KvTile<D, F8>& t, int k, int ok) {   // ok & 1 == 0: tile masked out
        const int bg = __builtin_amdgcn_readlane(tbg, k);
        const int j = __builtin_amdgcn_readlane(tj, k);
        if (bg != cur_bg) {
            if (cur_bg >= 0) end_piece();
            begin_piece(bg, j);
        }
        last_j = j;
        // A tile whose block id broke the precondition is read from block 0 and then
        // masked out entirely (arithmetic, not a branch, so every loaded register is
        // consumed and the waits stay per tile); an invalid second block (BS = 8) masks
        // rows 8-15.
        const int n = (ok & 1) ? ((ok & 2) ? seg_n : min(seg_n, j * 16 + 8)) : 0;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NQK; ++c) s = Mfma<T>::qk(k_operand<T, D>(t, c), qf[c], s);
        const int tok0 = j * 16 + 4 * quad;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = tok0 + e < n ? s[e] * a.scale_log2 : -INFINITY;
        const float bm = max_over_rows(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const bool move = bm > m + kSlack;
        if (__builtin_amdgcn_ballot_w64(move)) {
            const float mn = move ? bm : m;
            const float alpha = exp2_fast(m - mn);
            lsum *= alpha;
#pragma unroll
            for (int c = 0; c < NPV; ++c) acc[c] *= alpha;
            m = mn;
        }
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = x[e] == -INFINITY ? 0.f : exp2_fast(x[e] - m);
        lsum += (pe[0] + pe[1]) + (pe[2] + pe[3]);
        if (j * 16 + 16 > n) mask_rows<D>(t, tok0 + 0 < n, tok0 + 1 < n, tok0 + 2 < n, tok0 + 3 < n);
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) Mfma<T>::split(pe[e], hi[e], lo[e]);
        const uint2 phi = make_uint2(uint32_t(hi[0]) | (uint32_t(hi[1]) << 16),
                                     uint32_t(hi[2]) | (uint32_t(hi[3]) << 16));
        const uint2 plo = make_uint2(uint32_t(lo[0]) | (uint32_t(lo[1]) << 16),
                                     uint32_t(lo[2]) | (uint32_t(lo[3]) << 16));
#pragma unroll
        for (int c = 0; c < NPV; ++c) {
            const uint2 vv = v_operand<T, D>(t, c);
            acc[c] = Mfma<T>::pv(vv, phi, acc[c]);
            acc[c] = Mfma<T>::pv(vv, plo, acc[c]);
        }
    };

    // Batches of up to 64 tiles spanning up to kSplitPiecesPerBatch (b, g) pieces.
    // Per batch: lane k finds tile k's (b, g, j) by binary search, then the block ids
    // and the pieces' queries are fetched together (one wait), the queries staged in
    // this wave's LDS slots; the tiles then stream with no other load.
    for (int tb = t0; tb < t1;) {
        int cnt = min(64, t1 - tb);
        int lb = 0, lg = 0, lj = 0;
        if (lane < cnt) {
            const int t = tb + lane;
            int lo = 0, hi = a.num_seqs - 1;   // first b with s_end[b] > t
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_end[mid] > t) hi = mid; else lo = mid + 1;
            }
            const int nb = (s_len[lo] + 15) >> 4;
            const int r = t - (lo ? s_end[lo - 1] : 0);
            lb = lo;
            lg = r / nb;
            lj = r - lg * nb;
        }
        const int lbg = lb * hkv + lg;
        // lanes that open a new piece; cut the batch before the fifth one
        const int prev = __shfl_up(lbg, 1, 64);
        const bool opens = lane < cnt && (lane == 0 || prev != lbg);
        uint64_t opens_mask = __builtin_amdgcn_ballot_w64(opens);
        for (int c = 0; c < kSplitPiecesPerBatch && opens_mask; ++c) opens_mask &= opens_mask - 1;
        if (opens_mask) cnt = __builtin_ctzll(opens_mask);
        tbg = lbg;
        tj = lj;
        // One round trip for all metadata: the block ids of the batch and the queries
        // of its pieces (piece p opens at the p-th set bit of pm) are loaded together,
        // then the queries are staged in this wave's LDS slots.
        tile_ids<BS>(a.block_tables + int64_t(lb) * a.max_blocks, a.max_blocks,
                     lane < cnt ? lj : a.max_tiles, tphys, tphysb);
        const uint64_t pm = __builtin_amdgcn_ballot_w64(opens && lane < cnt);
        constexpr int kQChunks = (16 * D * 2 + 1023) / 1024;   // 1 KiB per lane-chunk, G <= 16
        uint4 qv[kSplitPiecesPerBatch][kQChunks];
        {
            uint64_t mm = pm;
#pragma unroll
            for (int p = 0; p < kSplitPiecesPerBatch; ++p) {
                const int src = mm ? __builtin_ctzll(mm) : 0;
                mm &= mm ? mm - 1 : 0;
                const int pbg = __builtin_amdgcn_readlane(lbg, src);
                const int pb = pbg / hkv, pg = pbg - pb * hkv;
                const uint16_t* qg = static_cast<const uint16_t*>(a.q) + int64_t(pb) * a.q_stride +
                                     int64_t(pg) * G * D;
#pragma unroll
                for (int c = 0; c < kQChunks; ++c) {
                    const int i = (c * 64 + lane) * 8;
                    qv[p][c] = i < qpiece ? *reinterpret_cast<const uint4*>(qg + i) : make_uint4(0, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int p = 0; p < kSplitPiecesPerBatch; ++p)
#pragma unroll
            for (int c = 0; c < kQChunks; ++c) {
                const int i = (c * 64 + lane) * 8;
                if (i < qpiece) *reinterpret_cast<uint4*>(my_q + p * qpiece + i) = qv[p][c];
            }
        piece_slot = -1;
        if (cur_bg >= 0 && __builtin_amdgcn_readlane(tbg, 0) == cur_bg) {
            // the batch continues the previous piece: keep its state, re-point the slot
            piece_slot = 0;
        }
        // FP8 tiles: two stages of kSplitStage tiles, the loads of the next stage issued
        // before the current one is used, so a wave keeps tiles in flight while it
        // computes. 16-bit tiles (8 KiB): one stage in flight per wave; on MI355X the 70B
        // batch took 308.8-313.5 us per launch against 313.1-319.7 with two (five calls
        // each, paired). Tiles past the end repeat the last one with every token masked:
        // the loop has no data-dependent branch, and each wait covers only the loads it
        // needs.
        constexpr int S = kSplitStage;   // also for FP8 tiles: stages of two measured slower
        KvTile<D, F8> X[S], Y[S];
        int okX[S], okY[S];
        auto load_stage = [&](KvTile<D, F8>* t, int* ok, int k) {
#pragma unroll
            for (int i = 0; i < S; ++i) ok[i] = load(t[i], min(k + i, cnt - 1));
        };
        auto compute_stage = [&](KvTile<D, F8>* t, const int* ok, int k) {
#pragma unroll
            for (int i = 0; i < S; ++i)
                compute(t[i], min(k + i, cnt - 1), k + i < cnt ? ok[i] : 0);
        };
        if constexpr (F8) {
            load_stage(X, okX, 0);
            for (int k = 0; k < cnt; k += 2 * S) {
                load_stage(Y, okY, k + S);
                compute_stage(X, okX, k);
                load_stage(X, okX, k + 2 * S);
                compute_stage(Y, okY, k + S);
            }
        } else {
            (void)Y;
            (void)okY;
            for (int k = 0; k < cnt; k += S) {
                load_stage(X, okX, k);
                compute_stage(X, okX, k);
            }
        }
        tb += cnt;
    }
    if (cur_bg >= 0) end_piece();
    flush();
}

// ---------------------------------------------------------------------- fp32
// 16-token blocks only. One wave per (partition, KV head, sequence). Lane l scores token l%16 for query
// heads l/16 and l/16 + 4 of the group; for the weighted sum it owns dimensions
// l and l + 64 of every head.
template <int D, typename OutT>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
    constexpr int GMAX = 8;
    constexpr int ND = (D + 63) / 64;
    __shared__ float sq[GMAX][D];
    __shared__ float sp[GMAX][16];
    __shared__ float salpha[GMAX];
    __shared__ float sm[1][16], sl[1][16];

    const int lane = threadIdx.x;
    const int g = a.heads_fastest ? blockIdx.x : blockIdx.y;
    const int b = a.heads_fastest ? blockIdx.y : blockIdx.z;
    const int p = a.heads_fastest ? blockIdx.z : blockIdx.x;
    const int G = a.group;
    int n = a.seq_lens[b];
    n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
    const int nblk = (n + 15) >> 4;
    const int blk_begin = p * a.part_tiles;
    if (blk_begin >= nblk) {
        if (p == 0) write_zero_rows<OutT, D>(a, b, g);
        return;
    }
    const int blk_end = min(nblk, blk_begin + a.part_tiles);
    const bool direct = nblk <= a.part_tiles;

    const float* qrow = static_cast<const float*>(a.q) + int64_t(b) * a.q_stride + int64_t(g) * G * D;
    for (int i = lane; i < G * D; i += 64) sq[i / D][i % D] = qrow[i];
    __syncthreads();

    const int t = lane & 15, hs = lane >> 4;
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    float acc[GMAX][ND];
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int k = 0; k < ND; ++k) acc[h][k] = 0.f;
    const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;
    const float* kbase = static_cast<const float*>(a.k_cache);
    const float* vbase = static_cast<const float*>(a.v_cache);
    for (int j = blk_begin; j < blk_end; ++j) {
        const int64_t phys = table[j];
        if (phys < 0 || phys >= a.num_blocks) continue;
        const int64_t tile = (phys * a.num_kv_heads + g) * int64_t(D) * 16;
        const float* kt = kbase + tile;   // [D/4][16][4]
        const float* vt = vbase + tile;   // [D][16]
        const bool valid = j * 16 + t < n;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int h = hs + 4 * r;
            float x = -INFINITY;
            if (h < G && valid) {
                float dot = 0.f;
                for (int i = 0; i < D; ++i) dot += sq[h][i] * kt[((i >> 2) * 16 + t) * 4 + (i & 3)];
                x = dot * a.scale_log2;
            }
            float bm = x;
#pragma unroll
            for (int s = 1; s < 16; s <<= 1) bm = wave_max_xor(bm, s);
            const float mn = fmaxf(m[r], bm);
            // a head with no valid token yet keeps -inf; guard the 0 * inf case
            const float alpha = mn == -INFINITY ? 1.f : exp2_fast(m[r] - mn);
            const float pv = x == -INFINITY ? 0.f : exp2_fast(x - mn);
            float ps = pv;
#pragma unroll
            for (int s = 1; s < 16; s <<= 1) ps += __shfl_xor(ps, s, 64);
            l[r] = l[r] * alpha + ps;
            m[r] = mn;
            if (h < G) {
                sp[h][t] = pv;
                if (t == 0) salpha[h] = alpha;
            }
        }
        __syncthreads();
        const int nvalid = min(16, n - j * 16);
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            if (h >= G) break;
            const float al = salpha[h];
#pragma unroll
            for (int k = 0; k < ND; ++k) {
                const int dim = lane + 64 * k;
                if (dim >= D) continue;
                float s = acc[h][k] * al;
                for (int tt = 0; tt < nvalid; ++tt) s += sp[h][tt] * vt[dim * 16 + tt];
                acc[h][k] = s;
            }
        }
        __syncthreads();
    }
    // publish each head's (m, l)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int h = hs + 4 * r;
        if (h < G && t == 0) {
            sm[0][h] = m[r];
            sl[0][h] = l[r];
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        if (h >= G) break;
        const float M = sm[0][h], L = sl[0][h];
        const int hq = g * G + h;
#pragma unroll
        for (int k = 0; k < ND; ++k) {
            const int dim = lane + 64 * k;
            if (dim >= D) continue;
            const float o = acc[h][k] / L;
            if (direct) {
                OutStore<OutT>::st(a.out, (int64_t(b) * a.num_heads + hq) * D + dim, o);
            } else {
                const int64_t row = (int64_t(b) * a.num_heads + hq) * a.max_partitions + p;
                a.part_out[row * D + dim] = o;
                if (dim == 0) {
                    a.part_max[row] = M * kLn2;
                    a.part_sum[row] = L;
                }
            }
        }
    }
}

// Waves per workgroup of the single-pass / partitioned kernels (4 or 8).
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
constexpr int kWaves = PKV_DECODE_WAVES;
static_assert(kWaves == 4 || kWaves == 8, "four or eight waves per workgroup");

template <typename T, int D, typename OutT, bool F8, int BS>
hipError_t launch_mfma(const DecodeArgs& a, dim3 grid, hipStream_t s) {
    const size_t lds = sizeof(float) * (2 * kWaves * 16 + size_t(kWaves) * a.group * D);
    const LaunchEvents ev = timer_events(PKV_TIMER_DECODE);
    if constexpr (BS == 32) {
        if (a.part_tiles % 2 == 0) {   // partitions of whole blocks: the whole-block kernel
            if (a.new_k)
                hipExtLaunchKernelGGL((decode_blk32_kernel<T, D, OutT, kWaves, true, F8>), grid,
                                      dim3(kWaves * 64), lds, s, ev.start, ev.stop, 0, a);
            else
                hipExtLaunchKernelGGL((decode_blk32_kernel<T, D, OutT, kWaves, false, F8>), grid,
                                      dim3(kWaves * 64), lds, s, ev.start, ev.stop, 0, a);
            return hipGetLastError();
        }
    }
    if (a.per_wave) {
        if (a.new_k)
            hipExtLaunchKernelGGL((decode_mfma_kernel<T, D, OutT, kWaves, true, F8, BS, true>), grid,
                                  dim3(kWaves * 64), lds, s, ev.start, ev.stop, 0, a);
        else
            hipExtLaunchKernelGGL((decode_mfma_kernel<T, D, OutT, kWaves, false, F8, BS, true>), grid,
                                  dim3(kWaves * 64), lds, s, ev.start, ev.stop, 0, a);
    } else if (a.new_k) {
        hipExtLaunchKernelGGL((decode_mfma_kernel<T, D, OutT, kWaves, true, F8, BS, false>), grid,
                              dim3(kWaves * 64), lds, s, ev.start, ev.stop, 0, a);
    } else {
        hipExtLaunchKernelGGL((decode_mfma_kernel<T, D, OutT, kWaves, false, F8, BS, false>), grid,
                              dim3(kWaves * 64), lds, s, ev.start, ev.stop, 0, a);
    }
    return hipGetLastError();
}

template <typename T, int D, typename OutT, bool F8, int BS>
hipError_t launch_split(const DecodeArgs& a, hipStream_t s) {
    const int groups = (a.split.units + kSplitThreads / 64 - 1) / (kSplitThreads / 64);
    const size_t lds = size_t(kSplitThreads / 64) * split_wave_bytes(a.group, D, a.slots);
    const LaunchEvents ev = timer_events(PKV_TIMER_DECODE);
    hipExtLaunchKernelGGL((decode_split_kernel<T, D, OutT, F8, BS>), dim3(groups),
                          dim3(kSplitThreads), lds, s, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

template <int D, typename OutT>
hipError_t launch_f32(const DecodeArgs& a, dim3 grid, hipStream_t s) {
    const LaunchEvents ev = timer_events(PKV_TIMER_DECODE);
    hipExtLaunchKernelGGL((decode_f32_kernel<D, OutT>), grid, dim3(64), 0, s, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

template <int D, bool F8, int BS>
hipError_t dispatch_16(const DecodeArgs& a, int in_dtype, int out_dtype, dim3 grid, hipStream_t s,
                       bool split) {
    if (split) {
        if (in_dtype == PKV_BF16)
            return out_dtype == PKV_F32 ? launch_split<bf16_t, D, float, F8, BS>(a, s)
                                        : launch_split<bf16_t, D, bf16_t, F8, BS>(a, s);
        return out_dtype == PKV_F32 ? launch_split<f16_t, D, float, F8, BS>(a, s)
                                    : launch_split<f16_t, D, f16_t, F8, BS>(a, s);
    }
    if (in_dtype == PKV_BF16)
        return out_dtype == PKV_F32 ? launch_mfma<bf16_t, D, float, F8, BS>(a, grid, s)
                                    : launch_mfma<bf16_t, D, bf16_t, F8, BS>(a, grid, s);
    return out_dtype == PKV_F32 ? launch_mfma<f16_t, D, float, F8, BS>(a, grid, s)
                                : launch_mfma<f16_t, D, f16_t, F8, BS>(a, grid, s);
}

// Launch the decode kernel for blocks of BS tokens (the fp32 kernel: BS = 16 only; the
// caller checks).
template <int BS>
hipError_t dispatch_bs(const DecodeArgs& a, int head_dim, int in_dtype, int out_dtype, dim3 grid,
                       hipStream_t s, bool split, bool fp8) {
    if (in_dtype == PKV_F32) {
        if constexpr (BS == 16)
            return head_dim == 128 ? launch_f32<128, float>(a, grid, s) : launch_f32<64, float>(a, grid, s);
        return hipErrorInvalidValue;
    }
    if (head_dim == 128)
        return fp8 ? dispatch_16<128, true, BS>(a, in_dtype, out_dtype, grid, s, split)
                   : dispatch_16<128, false, BS>(a, in_dtype, out_dtype, grid, s, split);
    return fp8 ? dispatch_16<64, true, BS>(a, in_dtype, out_dtype, grid, s, split)
               : dispatch_16<64, false, BS>(a, in_dtype, out_dtype, grid, s, split);
}

}  // namespace pkv
