// paged_attention_prefill: causal multi-query attention over the paged cache, for chunked
// prefill. A long prompt is processed in chunks over several steps; each chunk's K/V joins
// the cache (reshape_and_cache) and then its queries attend to every earlier position of
// the sequence and to the chunk up to themselves ("vLLM Nedir? PagedAttention ile
// Production LLM Serving", section "Chunked prefill"; "Yerel LLM sistemlerinde backpressure
// ve ölçekleme", section "4. Prefill ve decode"). With many queries per sequence the work
// is a dense contraction, so it runs on the matrix cores.
//
// Work decomposition: one workgroup of 8 waves per (query tile, KV head, sequence). The
// 16 columns of the matrix products are (query token, head of the GQA group) pairs; each
// wave owns NC column tiles of its own (16 * NC columns, 16 * NC / G query tokens), so a
// workgroup covers 8 * 16 * NC columns. The context is walked in stages of 64 keys that
// the workgroup stages in LDS once and all eight waves read: each K/V byte fetched from
// L2 feeds 8 * 16 * NC columns. (A design in which 4 waves shared one set of columns and
// split the keys fed each fetched byte to 16 * NC columns only; it needed about the whole
// L2 bandwidth to reach 23% of the matrix-core peak.) A stage is loaded into registers by
// all 512 threads while the previous one is computed, and written to the other of two LDS
// buffers after it: one barrier per stage. Each wave keeps its own online softmax per
// column and writes its rows itself. At two waves per SIMD (about 230 VGPRs) a CU holds
// one such workgroup; with 4 waves per workgroup (two per CU) each thread staged twice
// the bytes, and the kernel ran 8% slower.
//
// Per pair of 32 keys of a stage and column tile:
//   S_A^T, S_B^T[16 keys][16 cols] = K_rows x Q^T          (16x16x32, d/32 steps each)
//   O^T[d][16 cols] += V^T[d][32 keys] x P^T[32 keys][16 cols]   (16x16x32, d/16 steps)
// The two QK products read their K rows in a permuted order (row r of A: position
// 8 (r / 4) + r % 4 of the pair; of B: that + 4), so that lane l holds the logits of the
// 8 consecutive positions 8 (l/16) .. + 7, which are its 8 k-slots of the PV step in both
// operands: P stays in the lanes that produced it, and the lane's V operand is 8
// consecutive positions of one dimension row. The LDS layout is that of the operands,
// whatever the block size: K as [pair][product][16-byte dim group][MFMA row], V as
// [pair][8-key group][dim], so every operand read covers 128 contiguous bytes per 8 lanes,
// and the arithmetic (so the result) is the same for 8, 16 and 32 tokens per block.
//
// The weights enter the PV product once, rounded to fp16 (relative error at most 2^-11;
// they are 2^(x - m + 7) <= 2^15, so they reach fp16's subnormals only 21 binades below the
// column's maximum), and V enters it in fp16 too: a bf16 cache's V is converted as it is
// staged, which is exact for 2^-17 <= |v| <= 65,280 and moves smaller values by at most
// 2^-25. A bf16 V at or beyond 2^16 becomes +-inf, and every product with it (weight 0
// included) leaves the wave's accumulators non-finite; such a wave writes a NaN marker in
// place of its rows, and a second launch redoes those workgroups with the weights split in
// a high and a low bf16 part (two products, about 16 significant bits, as in decode). The
// same launch returns at once from every workgroup without a marker. With bf16 weights
// alone the error would reach about 3.7e-3 at a few keys and 1.7e-3 of max|out| at long
// contexts for N(0, 1) data; fp16 weights stay near 5e-4 and 2e-4.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
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
    float scale_log2;          // |scale| log2(e), at least the smallest normal float
    uint32_t q_sign;           // 0x80008000 when scale < 0: the queries' signs are flipped
};

constexpr int kPrefillWaves = 8;
constexpr int kPrefillNC = 2;       // column tiles per wave
// Keys per LDS stage (stage_keys / 32 pairs): 96 for head size 128, whose stage the 512
// threads load in exactly three 16-byte loads each (2% faster than 64 keys); 64 for head
// size 64 (one load each).
template <int D>
__host__ __device__ constexpr int stage_keys() { return D == 128 ? 96 : 64; }
constexpr float kSlack = 8.0f;      // lazy reference point, as in the decode kernel
constexpr float kPOffset = 7.0f;    // one-product form: weights 2^(x - m + 7) <= 2^15

// One LDS stage: K and V of 64 keys, D dims, 16-bit elements; two stages in flight.
template <int D>
__host__ __device__ constexpr size_t prefill_stage_bytes() {
    return size_t(2) * stage_keys<D>() * D * 2;
}
template <int D>
__host__ __device__ constexpr size_t prefill_lds_bytes() {
    return 2 * prefill_stage_bytes<D>();
}

// How the PV product takes the weights (see the header comment):
//   kSplitP: weights split into a high and a low part in the input type, two products;
//   kHalfP:  weights rounded once to fp16 and V in fp16 (a bf16 cache's V converted as it
//            is staged), one product; a wave whose accumulators end up non-finite writes a
//            NaN marker instead of its rows;
//   kRedo:   kSplitP, run only by workgroups whose rows carry such a marker.
constexpr int kSplitP = 0, kHalfP = 1, kRedo = 2;

// Two floats -> two fp16 (round to nearest even) in one word, lo in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

// acc + lo + hi of a word holding two fp16 values (one dot-product instruction, the two
// products with 1.0 exact, the sum rounded once to fp32).
__device__ __forceinline__ float sum_f16x2(uint32_t w, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), one, acc, false);
}

// Query tokens per wave: the 16 * NC columns hold whole tokens' G heads.
__host__ __device__ constexpr int prefill_wave_tokens(int G) { return 16 * kPrefillNC / G; }

// max of two logits, which are never NaN here (masked keys are -inf): the median of
// (a, b, +inf) is their maximum, and unlike fmaxf it needs no quieting of its inputs
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }
// max of three such logits in one instruction; written out because the compiler puts a
// quieting max in front of each operand of the max it would select itself
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// the maximum over the four lanes l % 16 + 16 k (the rows of one column)
__device__ __forceinline__ float rows_max(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = vmax(__builtin_bit_cast(float, (unsigned)r16[0]), __builtin_bit_cast(float, (unsigned)r16[1]));
    const unsigned w = __builtin_bit_cast(unsigned, y);
    auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return vmax(__builtin_bit_cast(float, (unsigned)r32[0]), __builtin_bit_cast(float, (unsigned)r32[1]));
}

// Element 0 of row `row` of out is NaN (the marker of a wave whose rows must be redone).
template <typename OutT> __device__ __forceinline__ bool marked(const void* out, int64_t row, int D);
template <> __device__ __forceinline__ bool marked<float>(const void* out, int64_t row, int D) {
    return __builtin_isnan(static_cast<const float*>(out)[row * D]);
}
template <> __device__ __forceinline__ bool marked<bf16_t>(const void* out, int64_t row, int D) {
    return (static_cast<const uint16_t*>(out)[row * D] & 0x7fff) > 0x7f80;
}
template <> __device__ __forceinline__ bool marked<f16_t>(const void* out, int64_t row, int D) {
    return (static_cast<const uint16_t*>(out)[row * D] & 0x7fff) > 0x7c00;
}

template <typename OutT> __device__ __forceinline__ void put_marker(void* out, int64_t row, int D) {
    if constexpr (std::is_same<OutT, float>::value)
        static_cast<uint32_t*>(out)[row * D] = 0x7fc00000u;
    else
        static_cast<uint16_t*>(out)[row * D] = std::is_same<OutT, bf16_t>::value ? 0x7fc0 : 0x7e00;
}

template <typename T, int D, typename OutT, int BS, int kMode>
__global__ __launch_bounds__(kPrefillWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(PrefillArgs a) {
    constexpr int W = kPrefillWaves, NC = kPrefillNC;
    constexpr int NQK = D / 32, NPV = D / 16;
    constexpr int NG = D / 8;                           // 16-byte K dim groups
    constexpr int kStageKeys = stage_keys<D>();
    constexpr int NLD = kStageKeys * D * 2 / 16 / (W * 64);   // 16-byte loads per thread, K and V each
    static_assert(NLD * 16 * W * 64 == kStageKeys * D * 2, "the threads' loads cover a stage exactly");
    constexpr int KCH = kStageKeys * NG;                // K chunks per stage
    constexpr int STAGE_CH = 2 * KCH;                   // K + V chunks per stage
    static_assert(NLD >= 1 && (NG * BS) % 64 == 0, "a load instruction stays in one block");
    extern __shared__ uint4 lds4[];                     // [2][STAGE_CH] 16-byte chunks

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int col = lane & 15, quad = lane >> 4;
    // KV heads fastest: consecutive workgroups go to the XCDs in turn, so (at 8 KV heads)
    // each XCD's L2 serves one head's K/V stages to all of its CUs, which walk the keys in
    // step (8% faster than query tiles fastest). Query tiles in reverse: under the causal
    // mask a later tile sees more keys, so the longest workgroups are dispatched first and
    // the short ones fill the tail.
    const int qt = int(gridDim.y) - 1 - int(blockIdx.y), g = blockIdx.x, b = blockIdx.z;
    const int G = a.group;
    const int TW = prefill_wave_tokens(G);              // query tokens per wave
    const int QT = W * TW;                              // per workgroup
    const int q0 = a.q_start[b];
    const int L = a.q_start[b + 1] - q0;
    const int t0 = qt * QT;
    if (t0 >= L) return;
    int n = a.seq_lens[b];
    n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
    const int tw0 = t0 + wave * TW;                     // this wave's first token
    // keys any query of the workgroup sees: up to the last valid token's position
    const int wg_last = min(QT, L - t0) - 1;
    if constexpr (kMode == kRedo) {
        // redo only a workgroup one of whose waves left its marker (element 0 of the row of
        // its first query token and the group's first head)
        bool redo = false;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const int tw = t0 + w * TW;
            if (tw < L) redo |= marked<OutT>(a.out, int64_t(q0 + tw) * a.num_heads + g * G, D);
        }
        if (!redo) return;
    }
    // the PV product's element type: fp16 in the one-product form
    using PV = typename std::conditional<kMode == kHalfP, f16_t, T>::type;
    constexpr bool kConvertV = kMode == kHalfP && std::is_same<T, bf16_t>::value;
    const int key_end = max(0, min(n, n - L + t0 + wg_last + 1));

    // This lane's column in each column tile: query token, head, causal limit (keys
    // below it are visible), and its Q^T operand.
    int lim[NC], tile_lim[NC], tile_min[NC];
    uint4 qf[NC][NQK];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        const int c = 16 * ct + col;
        const int tok = c / G, hg = c - tok * G;
        const bool valid = tok < TW && tw0 + tok < L;
        const int pos = n - L + tw0 + tok;               // the query's position in its sequence
        lim[ct] = valid ? max(0, min(pos + 1, n)) : 0;
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               int64_t(q0 + (valid ? tw0 + tok : 0)) * a.q_stride +
                               int64_t(g * G + hg) * D;
#pragma unroll
        for (int s = 0; s < NQK; ++s) {
            qf[ct][s] = valid ? *reinterpret_cast<const uint4*>(qrow + q_dim<false>(s, quad))
                              : make_uint4(0, 0, 0, 0);
            qf[ct][s].x ^= a.q_sign;
            qf[ct][s].y ^= a.q_sign;
            qf[ct][s].z ^= a.q_sign;
            qf[ct][s].w ^= a.q_sign;
        }
        int hi = lim[ct], lo = valid ? lim[ct] : 0x7fffffff;
#pragma unroll
        for (int k = 1; k < 16; k <<= 1) {
            hi = max(hi, __shfl_xor(hi, k, 64));
            lo = min(lo, __shfl_xor(lo, k, 64));
        }
        tile_lim[ct] = __builtin_amdgcn_readfirstlane(hi);   // largest limit of the tile
        tile_min[ct] = __builtin_amdgcn_readfirstlane(lo);   // smallest (valid columns)
    }
    int wave_end = 0;   // keys any column of this wave sees
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) wave_end = max(wave_end, tile_lim[ct]);

    f32x4 acc[NC][NPV];
    // m_ref: the column's reference point (log2 domain); nm: the offset its weights take,
    // -m_ref, or 0 while the column has seen no real key (m_ref = -inf), where every
    // logit is -inf too and the weights must stay 0 instead of exp2(-inf + inf)
    // thr = m_ref + kSlack; thr_raw = thr / scale_log2, against which each lane tests its
    // raw maximum (a lane past it leads to the exact test bm > thr)
    float m_ref[NC], nm[NC], thr[NC], thr_raw[NC], lsum[NC];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
#pragma unroll
        for (int c = 0; c < NPV; ++c) acc[ct][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_ref[ct] = -INFINITY;
        nm[ct] = 0.f;
        thr[ct] = -INFINITY;
        thr_raw[ct] = -INFINITY;
        lsum[ct] = 0.f;
    }

    // ---- stage loads: thread t issues load i of K and of V at linear chunk t + 256 i of
    // the stage, in the cache's own order (a block's K tile [NG][BS][16 B], then its V tile
    // [D][BS] as 16-byte runs of 8 positions), so consecutive lanes read consecutive
    // bytes; each instruction stays inside one block (a wave-uniform id). The chunk goes
    // to its place in the operand layout.
    const char* kbase = static_cast<const char*>(a.k_cache);
    const char* vbase = static_cast<const char*>(a.v_cache);
    const int64_t tile_bytes = int64_t(D) * BS * 2;     // one block of one KV head
    const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;
    const uint32_t nb_lim = block_limit(a.num_blocks);
    constexpr int SB = kStageKeys / BS;                 // blocks per stage
    const int tid = int(threadIdx.x);
    // ids of stage s's blocks: lane k < SB holds block k's (0 for an invalid or absent id:
    // a safe address; such rows break the precondition)
    auto stage_ids = [&](int s) {
        const int e = s * SB + lane;
        const int id = lane < SB && e < a.max_blocks ? table[e] : 0;
        return uint32_t(id) < nb_lim ? id : 0;
    };
    // native vectors, not uint4: copying the struct type between global, private and LDS
    // memory compiles to copies that keep the staging registers in scratch memory
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 kr[NLD], vr[NLD];
    auto issue = [&](int ids) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int lin = tid + W * 64 * i;
            const int bl = __builtin_amdgcn_readfirstlane(lin / (NG * BS));   // block in the stage
            const int within = lin - (lin / (NG * BS)) * (NG * BS);
            const int id = __builtin_amdgcn_readlane(ids, bl);
            const int64_t tb = (int64_t(id) * a.num_kv_heads + g) * tile_bytes;
            kr[i] = *reinterpret_cast<const u32x4*>(kbase + tb + int64_t(within) * 16);
            vr[i] = *reinterpret_cast<const u32x4*>(vbase + tb + int64_t(within) * 16);
        }
    };
    auto store = [&](uint4* dst) __attribute__((always_inline)) {
        u32x4* buf = reinterpret_cast<u32x4*>(dst);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int lin = tid + W * 64 * i;
            const int bl = lin / (NG * BS), within = lin - bl * (NG * BS);
            {   // K chunk: group gi, row -> key kl of the stage
                const int gi = within / BS, row = within - gi * BS;
                const int kl = bl * BS + row, m = kl >> 5, k32 = kl & 31;
                const int ab = (k32 >> 2) & 1, r = ((k32 >> 3) << 2) | (k32 & 3);
                buf[((m * 2 + ab) * NG + gi) * 16 + r] = kr[i];
            }
            {   // V chunk: dim d, 8 positions from row 8h -> 8-key group of the stage
                const int d = within / (BS / 8), h = within - d * (BS / 8);
                const int kl = bl * BS + 8 * h, m = kl >> 5, o = (kl & 31) >> 3;
                u32x4 vv = vr[i];
                if constexpr (kConvertV) {
                    // bf16 -> fp16, exact for 2^-17 <= |v| <= 65280; |v| >= 65536 becomes
                    // +-inf, which makes the accumulators of every column non-finite
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t u = vv[j];
                        vv[j] = pack_f16x2(__builtin_bit_cast(float, u << 16),
                                           __builtin_bit_cast(float, u & 0xffff0000u));
                    }
                }
                buf[KCH + (m * 4 + o) * D + d] = vv;
            }
        }
    };

    // ---- one pair of 32 keys (pair m of the stage in buf), both column tiles of the wave
    // in one block of straight-line code (one masking decision and one rescale branch per
    // pair), so that the scheduler can interleave one tile's softmax with the other's
    // matrix products. A tile whose queries see none of the pair goes through the masked
    // form, which gives it zero weights.
    auto load_k = [&](const uint4* buf, int m, uint4 (&ka)[NQK], uint4 (&kb)[NQK]) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < NQK; ++c) {
            ka[c] = buf[((m * 2 + 0) * NG + 4 * c + quad) * 16 + col];
            kb[c] = buf[((m * 2 + 1) * NG + 4 * c + quad) * 16 + col];
        }
    };
    auto compute_pair = [&](const uint4* buf, int kp, int m, uint4 (&ka)[NQK], uint4 (&kb)[NQK]) __attribute__((always_inline)) {
        uint4 v[NPV];
#pragma unroll
        for (int c = 0; c < NPV; ++c) v[c] = buf[KCH + (m * 4 + quad) * D + 16 * c + col];
        const int p0 = kp + 8 * quad;   // first of this lane's 8 positions
        // V rows past the sequence may hold anything: zeroed, only in a pair that has such
        // rows, so that their zero weights give zero products
        if (kp + 32 > n) {
            const int rn = n - p0;      // this lane's positions p0 + e with e < rn are valid
            auto keep = [&](int e) {
                return (e < rn ? 0x0000ffffu : 0u) | (e + 1 < rn ? 0xffff0000u : 0u);
            };
            const uint32_t k0 = keep(0), k1 = keep(2), k2 = keep(4), k3 = keep(6);
#pragma unroll
            for (int c = 0; c < NPV; ++c) {
                v[c].x &= k0;
                v[c].y &= k1;
                v[c].z &= k2;
                v[c].w &= k3;
            }
        }
        f32x4 sa[NC], sb[NC];
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            sa[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            sb[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NQK; ++c) {
                sa[ct] = Mfma<T>::qk(ka[c], qf[ct][c], sa[ct]);
                sb[ct] = Mfma<T>::qk(kb[c], qf[ct][c], sb[ct]);
            }
        }
        if (m + 1 < kStageKeys / 32) load_k(buf, m + 1, ka, kb);
        // raw logits (scale applied below): the causal diagonal, the sequence end and tiles
        // that see none of the pair take -inf per key
        bool masked = false;
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) masked |= kp + 32 > tile_min[ct] || kp >= tile_lim[ct];
        // lm: the maximum of this lane's 8 raw logits; the column's maximum is that of its
        // four lanes' lm, taken only when the reference point may move
        float x[NC][8], lm[NC];
        bool lane_move = false;
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[ct][e] = sa[ct][e];
                x[ct][4 + e] = sb[ct][e];
            }
            if (masked) {
                const int rem = lim[ct] - p0;   // positions p0 + e with e < rem are visible
#pragma unroll
                for (int e = 0; e < 8; ++e) x[ct][e] = e < rem ? x[ct][e] : -INFINITY;
            }
            const float t0 = vmax3(x[ct][0], x[ct][1], x[ct][2]);
            const float t1 = vmax3(x[ct][3], x[ct][4], x[ct][5]);
            const float t2 = vmax3(x[ct][6], x[ct][7], t0);
            lm[ct] = vmax3(t1, t2, t2);
            // while no lane passes, every visible x has x * scale <= thr * (1 + 2^-24), so the
            // weights stay within 2^15 to an ulp (thr_raw overflows to +inf only where no
            // finite x * scale can exceed thr)
            lane_move |= lm[ct] > thr_raw[ct];
        }
        if (__builtin_amdgcn_ballot_w64(lane_move)) {
#pragma unroll
            for (int ct = 0; ct < NC; ++ct) {
                // a column that keeps its reference keeps factor 1 (also one that has seen
                // no key yet, where m - m would be -inf - -inf)
                const float bm = rows_max(lm[ct]) * a.scale_log2;
                const bool move = bm > thr[ct];
                const float mn = move ? bm : m_ref[ct];
                const float alpha = move ? exp2_fast(m_ref[ct] - mn) : 1.0f;
                lsum[ct] *= alpha;
#pragma unroll
                for (int c = 0; c < NPV; ++c) acc[ct][c] *= alpha;
                m_ref[ct] = mn;
                nm[ct] = mn == -INFINITY ? 0.f : kPOffset - mn;
                thr[ct] = mn + kSlack;
                thr_raw[ct] = thr[ct] / a.scale_log2;
            }
        }
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            // 2^(x scale - m): 0 for x = -inf and a finite m
            float pe[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pe[e] = exp2_fast(__builtin_fmaf(x[ct][e], a.scale_log2, nm[ct]));
            if constexpr (kMode == kHalfP) {
                // one fp16 rounding per weight (weights in (2^-21, 2^15] before underflow);
                // the sum is of the same rounded weights, two per dot-product instruction
                const uint4 ph = make_uint4(pack_f16x2(pe[0], pe[1]), pack_f16x2(pe[2], pe[3]),
                                            pack_f16x2(pe[4], pe[5]), pack_f16x2(pe[6], pe[7]));
                lsum[ct] = sum_f16x2(ph.w, sum_f16x2(ph.z, sum_f16x2(ph.y, sum_f16x2(ph.x, lsum[ct]))));
#pragma unroll
                for (int c = 0; c < NPV; ++c) acc[ct][c] = Mfma<PV>::qk(v[c], ph, acc[ct][c]);
            } else {
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
                    acc[ct][c] = Mfma<T>::qk(v[c], phi, acc[ct][c]);
                    acc[ct][c] = Mfma<T>::qk(v[c], plo, acc[ct][c]);
                }
            }
        }
        if constexpr (kMode != kHalfP) {
            // split weights: tile 0's softmax, then tile 0's PV products one at a time
            // between tile 1's softmax instructions, then tile 1's PV products (measured
            // 1.5% faster than the compiler's order; slower for the one-product form)
            __builtin_amdgcn_sched_group_barrier(0x402, 48, 0);
#pragma unroll
            for (int i = 0; i < 2 * NPV; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * NPV, 0);
        }
    };

    // ---- the stages: stage s + 1 is in flight in registers while stage s is computed from
    // LDS, then written to the other buffer; one barrier per stage. The last stage loads
    // itself again into the unused buffer: with no condition around the loads and the
    // stores, the compiler keeps the staging registers in registers.
    const int S = (key_end + kStageKeys - 1) / kStageKeys;
    if (S > 0) {
        int ids = stage_ids(0);
        issue(ids);
        ids = stage_ids(min(1, S - 1));
        store(lds4);
        __syncthreads();
        // stage s reads buffer s % 2 and writes the other; the loop takes two stages per
        // iteration so that both buffers' addresses are constants folded into the LDS
        // instructions' offsets
        auto stage = [&](int s, auto parity) __attribute__((always_inline)) {
            constexpr int P = decltype(parity)::value;
            const uint4* cur = lds4 + P * STAGE_CH;
            issue(ids);                                 // stage min(s + 1, S - 1)
            ids = stage_ids(min(s + 2, S - 1));
            uint4 ka[NQK], kb[NQK];
            load_k(cur, 0, ka, kb);
#pragma unroll
            for (int m = 0; m < kStageKeys / 32; ++m) {
                const int kp = s * kStageKeys + 32 * m;
                if (kp < wave_end) compute_pair(cur, kp, m, ka, kb);
            }
            store(lds4 + (1 - P) * STAGE_CH);
            __syncthreads();
        };
        for (int s = 0; s < S; s += 2) {
            stage(s, std::integral_constant<int, 0>{});
            if (s + 1 < S) stage(s + 1, std::integral_constant<int, 1>{});
        }
    }

    if constexpr (kConvertV) {
        // a V element at or beyond 2^16 became +-inf in fp16, and every product with it
        // (weight 0 included) left this wave's accumulators non-finite (so would NaN or
        // infinite inputs, which the exact form then reproduces): the wave writes the
        // marker instead of its rows, and the kRedo pass computes them
        float sum = 0.f;
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
            for (int c = 0; c < NPV; ++c) sum += (acc[ct][c][0] + acc[ct][c][1]) + (acc[ct][c][2] + acc[ct][c][3]);
        if (__builtin_amdgcn_ballot_w64(!__builtin_isfinite(sum))) {
            if (lane == 0 && tw0 < L) put_marker<OutT>(a.out, int64_t(q0 + tw0) * a.num_heads + g * G, D);
            return;
        }
    }
    // ---- this wave's rows: lanes l, l^16, l^32, l^48 hold parts of the same column
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        float ls = lsum[ct];
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        const int c = 16 * ct + col;
        const int tok = c / G, hg = c - tok * G;
        if (tok >= TW || tw0 + tok >= L) continue;
        const int64_t row = int64_t(q0 + tw0 + tok) * a.num_heads + g * G + hg;
#pragma unroll
        for (int c2 = 0; c2 < NPV; ++c2) {
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);   // a query before position 0 sees no key
            if (ls > 0.f)
                o = make_float4(acc[ct][c2][0] / ls, acc[ct][c2][1] / ls, acc[ct][c2][2] / ls,
                                acc[ct][c2][3] / ls);
            OutStore<OutT>::st4(a.out, row * D + 16 * c2 + 4 * quad, o);
        }
    }
}

// One call: the one-product kernel, then (bf16 caches) the pass that redoes, in the exact
// split form, the workgroups whose waves met a V value beyond fp16's range; that pass's
// workgroups read a few marker elements and exit otherwise. The timer's events span both.
template <typename T, int D, typename OutT, int BS>
hipError_t launch_prefill(const PrefillArgs& a, int max_q_len, int num_kv_heads, int num_seqs,
                          hipStream_t s) {
    const int qt_tokens = kPrefillWaves * prefill_wave_tokens(a.group);
    const dim3 grid(unsigned(num_kv_heads), unsigned((max_q_len + qt_tokens - 1) / qt_tokens),
                    unsigned(num_seqs));
    const LaunchEvents ev = timer_events(PKV_TIMER_PREFILL);
    constexpr bool redo = std::is_same<T, bf16_t>::value;
    hipExtLaunchKernelGGL((prefill_kernel<T, D, OutT, BS, kHalfP>), grid, dim3(kPrefillWaves * 64),
                          prefill_lds_bytes<D>(), s, ev.start, redo ? nullptr : ev.stop, 0, a);
    hipError_t err = hipGetLastError();
    if constexpr (redo) {
        if (err != hipSuccess) return err;
        hipExtLaunchKernelGGL((prefill_kernel<T, D, OutT, BS, kRedo>), grid,
                              dim3(kPrefillWaves * 64), prefill_lds_bytes<D>(), s, nullptr, ev.stop,
                              0, a);
        err = hipGetLastError();
    }
    return err;
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
         reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out)) & 15)
        return fail(PKV_EINVAL, "%s: q, out and the caches must be 16-byte aligned", who);
    const int qt_tokens = pkv::kPrefillWaves * pkv::prefill_wave_tokens(G);
    if ((int64_t(max_q_len) + qt_tokens - 1) / qt_tokens > 65535)
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
    // the kernel takes the maximum of the raw logits and scales it, which needs a positive
    // scale: a negative one flips the queries' signs instead (exact), and a zero one is
    // raised to the smallest normal float (every weight still rounds to 1)
    const float sl2 = scale * 1.44269504088896340736f;
    a.scale_log2 = std::max(std::fabs(sl2), 1.17549435e-38f);
    a.q_sign = sl2 < 0.f ? 0x80008000u : 0u;
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
