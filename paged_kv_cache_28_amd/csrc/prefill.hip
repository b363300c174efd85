// paged_attention_prefill: causal multi-query attention over the paged cache, for chunked
// prefill. A long prompt is processed in chunks over several steps; each chunk's K/V joins
// the cache (reshape_and_cache) and then its queries attend to every earlier position of
// the sequence and to the chunk up to themselves ("vLLM Nedir? PagedAttention ile
// Production LLM Serving", section "Chunked prefill"; "Yerel LLM sistemlerinde backpressure
// ve ölçekleme", section "4. Prefill ve decode"). With many queries per sequence the work
// is a dense contraction, so it runs on the matrix cores.
//
// Work decomposition: one workgroup of 4 waves per (query tile, KV head, sequence). The
// 16 columns of the matrix products are (query token, head of the GQA group) pairs; a wave
// holds NC column tiles (16 * NC columns = 16 * NC / G query tokens), so every K/V pair it
// loads into registers feeds NC x 16 columns. The 4 waves take the key pairs round-robin
// with no barrier in the loop, each with its own online softmax per column, and merge
// through LDS one column tile at a time at the end. Causal mask: each lane masks with its
// own column's limit (keys at positions up to the query's), and a column tile whose queries
// see none of a pair skips it. (Staging the tiles in LDS for all four waves measured
// slower: the barrier per block kept the waves in lockstep.)
//
// Keys are walked in pairs of 32 consecutive positions, whatever the block size BS (8, 16
// or 32; a template parameter): a pair is four blocks, two blocks or one block. Per pair
// and column tile:
//   S_A^T, S_B^T[16 keys][16 cols] = K_rows x Q^T          (16x16x32, d/32 steps each)
//   O^T[d][16 cols] += V^T[d][32 keys] x P^T[32 keys][16 cols]   (16x16x32, d/16 steps)
// The two QK products read their K rows in a permuted order (row r of A: position
// 8 (r / 4) + r % 4 of the pair; of B: that + 4), so that lane l holds the logits of the
// 8 consecutive positions 8 (l/16) .. + 7, which are its 8 k-slots of the PV step in both
// operands: P stays in the lanes that produced it, and the lane's V operand is one 16-byte
// load of those positions of one dimension row. On gfx950 the 16x16x32 instruction issues
// at the rate of the 16x16x16 one with twice the work, so pairs halve the PV issue time. P
// is split in a high and a low bf16/fp16 part as in decode.
//
// Each pair is loaded and then used (no second pair in flight): with NC = 2 that keeps the
// wave at two per SIMD, and the other wave's math covers a pair's load. The vector-ALU work
// per pair bounds the kernel as much as anything (64 more multiplies per pair cost 7%), so
// the V rows past the real ones are zeroed once per pair and only in a pair that has any,
// and the softmax weights need no per-element select. Measured on the 30,000-token chunked
// prefill (TFLOP/s): this form 578-585; the masking per column tile and per element
// 544-547; two 16-token tiles W tiles apart with 8-byte V loads (24 loads per pair instead
// of 16) a further 1.5-3% less; the next pair's K and V loads issued into the same
// registers once the QK (resp. PV) products are done, no gain; double-buffered pairs (one
// wave per SIMD) 354; single blocks with the 16x16x16 product 460; NC = 1 (three waves per
// SIMD) 348; NC = 4 with Q^T in registers 361, in LDS 531 (against 540); tiles staged in
// LDS for the workgroup 290.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "device.hpp"
#include "status.hpp"
#include "tile.hpp"
#include "timer.hpp"

namespace pkv {

struct PrefillArgs {
    void* out;                 // [T][Hq][D]
    const void* q;             // row r at q + r * q_stride
    const int32_t* q_start;    // [num_seqs + 1]
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    int64_t q_stride;
    int64_t num_blocks;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t max_blocks;
    int32_t max_len;           // max_blocks * block size
    int32_t max_tiles;         // ceil(max_len / 16)
    float scale_log2;
};

constexpr int kPrefillWaves = 4;

template <int D>
__host__ __device__ constexpr size_t prefill_lds_bytes() {
    return sizeof(float) * (2 * kPrefillWaves * 16 + size_t(kPrefillWaves) * 16 * D);
}

template <typename T, int D, typename OutT, int NC, int BS>
__global__ __launch_bounds__(kPrefillWaves * 64) void prefill_kernel(PrefillArgs a) {
    constexpr int W = kPrefillWaves;
    constexpr int NQK = D / 32, NPV = D / 16;
    extern __shared__ float lds[];
    float* sm_m = lds;                  // [W][16]
    float* sm_l = lds + W * 16;         // [W][16]
    float* sm_o = lds + 2 * W * 16;     // [W][16][D]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, quad = lane >> 4;
    // query tiles in reverse: under the causal mask a later tile sees more keys, so the
    // longest workgroups are dispatched first and the short ones fill the tail
    const int qt = int(gridDim.x) - 1 - int(blockIdx.x), g = blockIdx.y, b = blockIdx.z;
    const int G = a.group;
    const int QT = 16 * NC / G;         // query tokens of this workgroup
    const int q0 = a.q_start[b];
    const int L = a.q_start[b + 1] - q0;
    const int t0 = qt * QT;
    if (t0 >= L) return;
    const int tcount = min(QT, L - t0);
    int n = a.seq_lens[b];
    n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);

    // This lane's column in each column tile: query token, head, causal limit (keys
    // below it are visible), and its Q^T operand.
    int lim[NC];
    int tile_lim[NC];   // largest limit of the column tile (wave-uniform)
    uint4 qf[NC][NQK];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        const int c = 16 * ct + col;
        const int tok = c / G, hg = c - tok * G;
        const bool valid = tok < tcount;
        const int pos = n - L + t0 + tok;          // the query's position in its sequence
        lim[ct] = valid ? max(0, min(pos + 1, n)) : 0;
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               int64_t(q0 + t0 + (valid ? tok : 0)) * a.q_stride +
                               int64_t(g * G + hg) * D;
#pragma unroll
        for (int s = 0; s < NQK; ++s)
            qf[ct][s] = valid ? *reinterpret_cast<const uint4*>(qrow + q_dim<false>(s, quad))
                              : make_uint4(0, 0, 0, 0);
        int m = lim[ct];
#pragma unroll
        for (int k = 1; k < 16; k <<= 1) m = max(m, __shfl_xor(m, k, 64));
        tile_lim[ct] = __builtin_amdgcn_readfirstlane(m);
    }
    int key_end = 0;   // keys any column of the workgroup sees
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) key_end = max(key_end, tile_lim[ct]);

    f32x4 acc[NC][NPV];
    float m_ref[NC], lsum[NC];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
#pragma unroll
        for (int c = 0; c < NPV; ++c) acc[ct][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_ref[ct] = -INFINITY;
        lsum[ct] = 0.f;
    }
    constexpr float kSlack = 8.0f;   // lazy reference point, as in the decode kernel

    const char* kbase = static_cast<const char*>(a.k_cache);
    const char* vbase = static_cast<const char*>(a.v_cache);
    const int64_t tile_bytes = int64_t(D) * BS * 2;   // one block of one KV head
    const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;

    // Keys are walked in pairs of 32 consecutive positions (pair m: 32m .. 32m + 31, the
    // 16-token tiles 2m and 2m + 1), each a 16x16x32 PV step. The QK products read their
    // K rows in a permuted order so that each lane ends up holding the logits of 8
    // consecutive positions: MFMA row r of product A reads position 8 (r / 4) + r % 4 of
    // the pair, product B that position + 4, so lane (quad, col) gets positions
    // 8 quad .. 8 quad + 3 from A and 8 quad + 4 .. + 7 from B. Its V operand is then one
    // 16-byte load of those 8 positions of one dimension row, half the V loads of two
    // 16-token tiles. 8 consecutive positions never cross a block (BS >= 8).
    constexpr int NB = 32 / BS;                         // blocks per pair (4, 2, 1)
    const int ra = 8 * (col >> 2) + (col & 3), rb = ra + 4, rv = 8 * quad;
    auto blk_of = [](int t) { return t / BS; };
    auto row_of = [](int t) { return t % BS; };
    int ids[NB];   // block ids of this segment: lane k holds pair k's

    struct Pair {
        uint4 ka[NQK];   // K rows of product A, QK steps 0 .. NQK - 1
        uint4 kb[NQK];   // product B
        uint4 v[NPV];    // positions 8 quad .. + 7 of dimension 16 c + col
    };

    // Issue the loads of segment pair k. Returns bit i set if the pair's block i has a
    // valid id; an invalid id is replaced by a safe address and its rows masked.
    auto load_pair = [&](Pair& t, int k) __attribute__((always_inline)) -> int {
        int okm = 0;
        auto id = [&](int i) -> int32_t {   // block i's id, or 0 (safe) if invalid
            const int32_t p = __builtin_amdgcn_readlane(ids[i], k);
            const bool ok = p >= 0 && int64_t(p) < a.num_blocks;
            okm |= int(ok) << i;
            return ok ? p : 0;
        };
        // separate variables, not an array: the compiler turns selects among array
        // elements into an indexed scratch access
        const int32_t p0 = id(0);
        const int32_t p1 = NB > 1 ? id(1) : 0;
        const int32_t p2 = NB > 2 ? id(2) : 0;
        const int32_t p3 = NB > 2 ? id(3) : 0;
        auto pick = [&](int bi) {   // the id of pair block bi (lane-varying)
            const int32_t lo = (bi & 1) ? p1 : p0;
            const int32_t hi = (bi & 1) ? p3 : p2;
            const int32_t p = NB == 1 ? p0 : NB == 2 ? lo : ((bi & 2) ? hi : lo);
            return (int64_t(p) * a.num_kv_heads + g) * tile_bytes;
        };
        const char* kA = kbase + pick(blk_of(ra));
        const char* kB = kbase + pick(blk_of(rb));
        const char* vt = vbase + pick(blk_of(rv));
        const int rowa = row_of(ra), rowb = row_of(rb), rowv = row_of(rv);
#pragma unroll
        for (int c = 0; c < NQK; ++c) {
            t.ka[c] = *reinterpret_cast<const uint4*>(kA + ((4 * c + quad) * BS + rowa) * 16);
            t.kb[c] = *reinterpret_cast<const uint4*>(kB + ((4 * c + quad) * BS + rowb) * 16);
        }
#pragma unroll
        for (int c = 0; c < NPV; ++c)
            t.v[c] = *reinterpret_cast<const uint4*>(vt + ((16 * c + col) * BS + rowv) * 2);
        return okm;
    };

    auto compute_pair = [&](Pair& t, int m, int okm) __attribute__((always_inline)) {
        const int p0 = 32 * m + 8 * quad;   // first of this lane's 8 positions
        // positions below nv are real: past the sequence, or in a block whose id is
        // invalid, they are not
        const int nv = ((okm >> blk_of(rv)) & 1) ? n : 0;
        // V rows that are not real may hold anything: zeroed once per pair, and only in a
        // pair that has such rows (the last pair of a sequence or an invalid block)
        if (__builtin_amdgcn_ballot_w64(p0 + 8 > nv)) {
            auto keep = [&](int q) {
                return (q < nv ? 0x0000ffffu : 0u) | (q + 1 < nv ? 0xffff0000u : 0u);
            };
            const uint32_t k0 = keep(p0), k1 = keep(p0 + 2), k2 = keep(p0 + 4), k3 = keep(p0 + 6);
#pragma unroll
            for (int c = 0; c < NPV; ++c) {
                t.v[c].x &= k0;
                t.v[c].y &= k1;
                t.v[c].z &= k2;
                t.v[c].w &= k3;
            }
        }
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            if (32 * m >= tile_lim[ct]) continue;   // no query of this tile sees the pair
            const int lv = min(lim[ct], nv);
            f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NQK; ++c) {
                sa = Mfma<T>::qk(t.ka[c], qf[ct][c], sa);
                sb = Mfma<T>::qk(t.kb[c], qf[ct][c], sb);
            }
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = p0 + e < lv ? sa[e] * a.scale_log2 : -INFINITY;
                x[4 + e] = p0 + 4 + e < lv ? sb[e] * a.scale_log2 : -INFINITY;
            }
            const float bm = max_over_rows(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                                 fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
            const bool move = bm > m_ref[ct] + kSlack;
            if (__builtin_amdgcn_ballot_w64(move)) {
                // a lane that keeps its reference keeps factor 1 (also one whose column has
                // seen no key yet, where m - m would be -inf - -inf)
                const float mn = move ? bm : m_ref[ct];
                const float alpha = move ? exp2_fast(m_ref[ct] - mn) : 1.0f;
                lsum[ct] *= alpha;
#pragma unroll
                for (int c = 0; c < NPV; ++c) acc[ct][c] *= alpha;
                m_ref[ct] = mn;
            }
            // exp2(-inf - m) is 0 for a finite m; m is -inf only while the column has seen
            // no real key, and then every x is -inf too, so one select per lane (not per
            // element) keeps those weights 0 instead of exp2(-inf + inf)
            const float mref = m_ref[ct] == -INFINITY ? 0.f : m_ref[ct];
            float pe[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pe[e] = exp2_fast(x[e] - mref);
            lsum[ct] += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
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
                acc[ct][c] = Mfma<T>::qk(t.v[c], phi, acc[ct][c]);
                acc[ct][c] = Mfma<T>::qk(t.v[c], plo, acc[ct][c]);
            }
        }
    };

    // This wave's pairs: wave, wave + W, ...; segments of 64 pairs (block ids one pair per
    // lane), each pair loaded and then used.
    const int npairs = (key_end + 31) >> 5;
    const int nmine = wave < npairs ? (npairs - wave + W - 1) / W : 0;
    for (int k0 = 0; k0 < nmine; k0 += 64) {
        const int cnt = min(64, nmine - k0);
        const int mp = wave + (k0 + lane) * W;   // this lane's pair
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int bi = NB * mp + i;
            ids[i] = lane < cnt && bi < a.max_blocks ? table[bi] : -1;
        }
        for (int k = 0; k < cnt; ++k) {
            Pair t;
            const int okm = load_pair(t, k);
            compute_pair(t, wave + (k0 + k) * W, okm);
        }
    }

    // Merge the waves' states column tile by column tile and write the rows.
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        float ls = lsum[ct];
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        if (lane < 16) {
            sm_m[wave * 16 + lane] = m_ref[ct];
            sm_l[wave * 16 + lane] = ls;
        }
#pragma unroll
        for (int c = 0; c < NPV; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) sm_o[(wave * 16 + col) * D + 16 * c + 4 * quad + e] = acc[ct][c][e];
        __syncthreads();
        for (int i = threadIdx.x; i < 16 * D; i += W * 64) {
            const int c = i / D, dim = i - c * D;
            const int cc = 16 * ct + c;
            const int tok = cc / G, hg = cc - tok * G;
            if (tok >= tcount) continue;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w * 16 + c]);
            float o = 0.f;
            if (M != -INFINITY) {   // a query before position 0 sees no key: zero row
                float Lw = 0.f, O = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const float f = exp2_fast(sm_m[w * 16 + c] - M);
                    Lw += f * sm_l[w * 16 + c];
                    O += f * sm_o[(w * 16 + c) * D + dim];
                }
                o = O / Lw;
            }
            const int64_t row = int64_t(q0 + t0 + tok) * a.num_heads + g * G + hg;
            OutStore<OutT>::st(a.out, row * D + dim, o);
        }
        __syncthreads();
    }
}

template <typename T, int D, typename OutT, int BS>
hipError_t launch_prefill(const PrefillArgs& a, int max_q_len, int num_kv_heads, int num_seqs,
                          hipStream_t s) {
    constexpr int NC = 2;
    const int qt_tokens = 16 * NC / a.group;
    const dim3 grid(unsigned((max_q_len + qt_tokens - 1) / qt_tokens), unsigned(num_kv_heads),
                    unsigned(num_seqs));
    const LaunchEvents ev = timer_events(PKV_TIMER_PREFILL);
    hipExtLaunchKernelGGL((prefill_kernel<T, D, OutT, NC, BS>), grid, dim3(kPrefillWaves * 64),
                          prefill_lds_bytes<D>(), s, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

template <int BS>
hipError_t dispatch_prefill(const PrefillArgs& a, int head_dim, int in_dtype, int out_dtype,
                            int max_q_len, int num_kv_heads, int num_seqs, hipStream_t s) {
    const bool f32 = out_dtype == PKV_F32;
    if (head_dim == 128) {
        if (in_dtype == PKV_BF16)
            return f32 ? launch_prefill<bf16_t, 128, float, BS>(a, max_q_len, num_kv_heads, num_seqs, s)
                       : launch_prefill<bf16_t, 128, bf16_t, BS>(a, max_q_len, num_kv_heads, num_seqs, s);
        return f32 ? launch_prefill<f16_t, 128, float, BS>(a, max_q_len, num_kv_heads, num_seqs, s)
                   : launch_prefill<f16_t, 128, f16_t, BS>(a, max_q_len, num_kv_heads, num_seqs, s);
    }
    if (in_dtype == PKV_BF16)
        return f32 ? launch_prefill<bf16_t, 64, float, BS>(a, max_q_len, num_kv_heads, num_seqs, s)
                   : launch_prefill<bf16_t, 64, bf16_t, BS>(a, max_q_len, num_kv_heads, num_seqs, s);
    return f32 ? launch_prefill<f16_t, 64, float, BS>(a, max_q_len, num_kv_heads, num_seqs, s)
               : launch_prefill<f16_t, 64, f16_t, BS>(a, max_q_len, num_kv_heads, num_seqs, s);
}

}  // namespace pkv

extern "C" int paged_attention_prefill(void* out, const void* q, int64_t q_stride,
                                       const int32_t* q_start, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t max_q_len, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                       int32_t in_dtype, int32_t out_dtype, void* stream) {
    using pkv::fail;
    const char* who = "paged_attention_prefill";
    if (in_dtype != PKV_F16 && in_dtype != PKV_BF16)
        return fail(in_dtype == PKV_F32 ? PKV_ENOTSUP : PKV_EINVAL,
                    "%s: in_dtype must be F16 or BF16", who);
    if (out_dtype != in_dtype && out_dtype != PKV_F32)
        return fail(PKV_ENOTSUP, "%s: out_dtype must be in_dtype or F32", who);
    if (num_seqs < 0 || max_q_len < 0) return fail(PKV_EINVAL, "%s: negative sizes", who);
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PKV_EINVAL, "%s: block_size must be 8, 16 or 32, got %d", who, block_size);
    if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
        return fail(PKV_EINVAL, "%s: num_heads %d not a multiple of num_kv_heads %d", who,
                    num_heads, num_kv_heads);
    if (num_seqs > 65535 || num_kv_heads > 65535)
        return fail(PKV_EINVAL, "%s: num_seqs / num_kv_heads above 65535", who);
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_ENOTSUP, "%s: head_dim %d (built: 64, 128)", who, head_dim);
    const int G = num_heads / num_kv_heads;
    if (G > 16) return fail(PKV_ENOTSUP, "%s: group size %d too large", who, G);
    if (max_blocks_per_seq <= 0 || num_blocks <= 0 ||
        int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
        return fail(PKV_EINVAL, "%s: bad max_blocks_per_seq / num_blocks", who);
    if (q_stride < int64_t(num_heads) * head_dim || q_stride % 8)
        return fail(PKV_EINVAL, "%s: q_stride must cover num_heads*head_dim and be a multiple "
                                "of 8", who);
    if (!std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale not finite", who);
    if (num_seqs == 0 || max_q_len == 0) return pkv::ok();
    if (!out || !q || !q_start || !k_cache || !v_cache || !block_tables || !seq_lens)
        return fail(PKV_EINVAL, "%s: NULL pointer", who);
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
         reinterpret_cast<uintptr_t>(v_cache)) & 15)
        return fail(PKV_EINVAL, "%s: q and caches must be 16-byte aligned", who);
    const int qt_tokens = 16 * 2 / G;
    if ((int64_t(max_q_len) + qt_tokens - 1) / qt_tokens > 0x7fffffff)
        return fail(PKV_EINVAL, "%s: max_q_len too large", who);
    pkv::PrefillArgs a;
    a.out = out;
    a.q = q;
    a.q_start = q_start;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.q_stride = q_stride;
    a.num_blocks = num_blocks;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = G;
    a.max_blocks = max_blocks_per_seq;
    a.max_len = max_blocks_per_seq * block_size;
    a.max_tiles = (a.max_len + 15) / 16;
    a.scale_log2 = scale * 1.44269504088896340736f;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err =
        block_size == 16
            ? pkv::dispatch_prefill<16>(a, head_dim, in_dtype, out_dtype, max_q_len, num_kv_heads, num_seqs, s)
        : block_size == 8
            ? pkv::dispatch_prefill<8>(a, head_dim, in_dtype, out_dtype, max_q_len, num_kv_heads, num_seqs, s)
            : pkv::dispatch_prefill<32>(a, head_dim, in_dtype, out_dtype, max_q_len, num_kv_heads, num_seqs, s);
    if (err != hipSuccess)
        return fail(PKV_EHIP, "%s: launch failed: %s", who, hipGetErrorString(err));
    return pkv::ok();
}
