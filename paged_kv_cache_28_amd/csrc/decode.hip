// paged_attention_decode and its variants (fused append, FP8 cache): argument checks,
// launch planning and the entry points. The kernels are in decode_kernels.hpp; this unit
// instantiates them for 16-token blocks, decode_bs8.hip and decode_bs32.hip for 8 and 32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <numeric>
#include <vector>

#include "decode_kernels.hpp"

namespace pkv {

template hipError_t dispatch_bs<16>(const DecodeArgs&, int, int, int, dim3, hipStream_t, bool, bool);
extern template hipError_t dispatch_bs<8>(const DecodeArgs&, int, int, int, dim3, hipStream_t, bool, bool);
extern template hipError_t dispatch_bs<32>(const DecodeArgs&, int, int, int, dim3, hipStream_t, bool, bool);

int device_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

// Waves per compute unit that the balanced split plans for: two workgroups of four
// waves (two waves per SIMD) on every unit. With two tiles in flight per wave this keeps
// enough reads queued to saturate HBM; deeper queues measured slower (the extra reads
// only add queueing delay and spread the finishing times of the waves).
// PKV_SPLIT_WAVES_PER_CU overrides the count (a tuning knob; it must not change between
// a decode and its reduce).
int split_units() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int per = 8;
        if (const char* env = std::getenv("PKV_SPLIT_WAVES_PER_CU")) {
            const int v = std::atoi(env);
            if (v > 0 && v <= 64) per = v;
        }
        cache[dev] = device_cus() * per;
    }
    return cache[dev];
}

}  // namespace pkv

namespace {

// The new tokens of a fused append (null key: plain decode).
struct AppendIn {
    const void* key;
    const void* value;
    int64_t key_stride;
    int64_t value_stride;
    const int32_t* slot_mapping;
};

// FP8 cache: kv_dtype == PKV_FP8_E4M3 and its two scales; otherwise kv_dtype == in_dtype.
int decode_impl(const char* who, void* out, float* part_out, float* part_max, float* part_sum,
                const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                int32_t partition_size, int32_t max_partitions, int32_t in_dtype,
                int32_t out_dtype, int32_t kv_dtype, float k_scale, float v_scale,
                const AppendIn& app, const int32_t* seq_order, void* stream) {
    using pkv::fail;
    const int e = pkv::elem_bytes(in_dtype);
    if (e == 0) return fail(PKV_EINVAL, "%s: unknown in_dtype %d", who, in_dtype);
    const bool fp8 = kv_dtype == PKV_FP8_E4M3;
    if (fp8) {
        if (in_dtype == PKV_F32)
            return fail(PKV_ENOTSUP, "%s: an FP8 cache needs F16 or BF16 queries", who);
        if (!(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
            return fail(PKV_EINVAL, "%s: k_scale and v_scale must be finite and positive", who);
    } else {
        k_scale = v_scale = 1.0f;
    }
    if (pkv::elem_bytes(out_dtype) == 0)
        return fail(PKV_EINVAL, "%s: unknown out_dtype %d", who, out_dtype);
    if (out_dtype != in_dtype && out_dtype != PKV_F32)
        return fail(PKV_ENOTSUP, "%s: out_dtype must be in_dtype or F32", who);
    if (num_seqs < 0) return fail(PKV_EINVAL, "%s: negative num_seqs", who);
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PKV_EINVAL, "%s: block_size must be 8, 16 or 32, got %d", who, block_size);
    if (in_dtype == PKV_F32 && block_size != 16)
        return fail(PKV_ENOTSUP, "%s: fp32 inputs need 16-token blocks", who);
    if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
        return fail(PKV_EINVAL, "%s: num_heads %d not a multiple of "
                                "num_kv_heads %d", who, num_heads, num_kv_heads);
    if (num_seqs > 65535 || num_kv_heads > 65535)
        return fail(PKV_EINVAL, "%s: num_seqs / num_kv_heads above 65535", who);
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_ENOTSUP, "%s: head_dim %d (built: 64, 128)", who, head_dim);
    const int G = num_heads / num_kv_heads;
    if ((in_dtype == PKV_F32 && G > 8) || G > 16)
        return fail(PKV_ENOTSUP, "%s: group size %d too large", who, G);
    if (max_blocks_per_seq <= 0 || num_blocks <= 0 ||
        int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
        return fail(PKV_EINVAL, "%s: bad max_blocks_per_seq / num_blocks", who);
    // the context is walked in 16-token tiles whatever the block size
    const int32_t max_len = max_blocks_per_seq * block_size;
    const int32_t max_tiles = (max_len + 15) / 16;
    const int x = 16 / e;
    if (q_stride < int64_t(num_heads) * head_dim || q_stride % x)
        return fail(PKV_EINVAL, "%s: q_stride must cover num_heads*head_dim "
                                "and be a multiple of %d", who, x);
    if (!std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale not finite", who);
    int part_tiles = max_tiles, grid_parts = 1;
    const bool split = partition_size == PKV_PARTITION_AUTO;
    if (!split && (partition_size < 0 || partition_size % 16))
        return fail(PKV_EINVAL, "%s: partition_size must be 0, "
                                "PKV_PARTITION_AUTO or a positive multiple of 16", who);
    if (split) {
        if (in_dtype == PKV_F32)
            return fail(PKV_ENOTSUP, "%s: PKV_PARTITION_AUTO needs fp16/bf16", who);
        if (num_seqs > pkv::kSplitMaxSeqs)
            return fail(PKV_ENOTSUP, "%s: PKV_PARTITION_AUTO takes at most %d "
                                     "sequences", who, pkv::kSplitMaxSeqs);
        if (int64_t(num_seqs) * num_kv_heads * max_tiles >= (int64_t(1) << 31))
            return fail(PKV_ENOTSUP, "%s: too many tiles for PKV_PARTITION_AUTO", who);
        if (max_partitions < 2)
            return fail(PKV_EINVAL, "%s: PKV_PARTITION_AUTO needs "
                                    "max_partitions >= 2", who);
        grid_parts = 2;   // partial buffers are required below
    } else if (partition_size > 0) {
        part_tiles = partition_size / 16;
        grid_parts = (max_tiles + part_tiles - 1) / part_tiles;
        if (max_partitions < grid_parts)
            return fail(PKV_EINVAL, "%s: max_partitions %d < %d", who,
                        max_partitions, grid_parts);

    }
    if (num_seqs == 0) return pkv::ok();
    if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens)
        return fail(PKV_EINVAL, "%s: NULL pointer", who);
    if (seq_order) {   // host memory: a permutation of the batch
        std::vector<char> seen(size_t(num_seqs), 0);
        for (int32_t i = 0; i < num_seqs; ++i) {
            const int32_t v = seq_order[i];
            if (v < 0 || v >= num_seqs || seen[size_t(v)])
                return fail(PKV_EINVAL, "%s: seq_order is not a permutation of the batch", who);
            seen[size_t(v)] = 1;
        }
    }
    if (grid_parts > 1 && (!part_out || !part_max || !part_sum))
        return fail(PKV_EINVAL, "%s: partitioned mode needs part_* buffers", who);
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
         reinterpret_cast<uintptr_t>(v_cache)) & 15)
        return fail(PKV_EINVAL, "%s: q and caches must be 16-byte aligned", who);
    if (split && ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(part_out)) & 15))
        return fail(PKV_EINVAL, "%s: PKV_PARTITION_AUTO needs 16-byte "
                                "aligned out and part_out", who);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Fused append: validated like reshape_and_cache. The fp32 and balanced-split kernels
    // take it as a cache-write launch ahead of the decode launch (same result).
    bool fused = false;
    if (app.key) {
        if (!app.value || !app.slot_mapping)
            return fail(PKV_EINVAL, "%s: NULL key/value/slot_mapping", who);
        if (app.key_stride < int64_t(num_kv_heads) * head_dim ||
            app.value_stride < int64_t(num_kv_heads) * head_dim || app.key_stride % x ||
            app.value_stride % x)
            return fail(PKV_EINVAL, "%s: key/value sequence strides must cover "
                                    "num_kv_heads*head_dim and be multiples of %d", who, x);
        if ((reinterpret_cast<uintptr_t>(app.key) | reinterpret_cast<uintptr_t>(app.value)) & 15)
            return fail(PKV_EINVAL, "%s: key and value must be 16-byte aligned", who);
        fused = in_dtype != PKV_F32 && !split;
        if (!fused) {
            const int rc =
                fp8 ? reshape_and_cache_fp8(app.key, app.value, const_cast<void*>(k_cache),
                                            const_cast<void*>(v_cache), app.slot_mapping, num_seqs,
                                            num_kv_heads, head_dim, block_size, num_blocks,
                                            app.key_stride, app.value_stride, in_dtype, k_scale,
                                            v_scale, stream)
                    : reshape_and_cache(app.key, app.value, const_cast<void*>(k_cache),
                                        const_cast<void*>(v_cache), app.slot_mapping, num_seqs,
                                        num_kv_heads, head_dim, block_size, num_blocks,
                                        app.key_stride, app.value_stride, in_dtype, stream);
            if (rc != PKV_OK) return rc;
        }
    }

    pkv::DecodeArgs a;
    a.out = out;
    a.part_out = part_out;
    a.part_max = part_max;
    a.part_sum = part_sum;
    a.q = q;
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
    a.max_len = max_len;
    a.max_tiles = max_tiles;
    a.part_tiles = part_tiles;
    a.max_partitions = partition_size != 0 ? max_partitions : 1;
    a.scale_log2 = scale * k_scale * pkv::kLog2e;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.num_seqs = num_seqs;
    a.split.units = split ? pkv::split_units() : 0;
    a.split.min_share = split ? (max_tiles + max_partitions - 2) / (max_partitions - 1) : 0;
    {
        const int slot_bytes = pkv::split_slot_floats(G, head_dim) * 4 + 16;
        const int room = pkv::kSplitWaveLds - pkv::split_q_bytes(G, head_dim);
        a.slots = std::min(pkv::kSplitMaxSlots, std::max(1, room / slot_bytes));
    }
    a.new_k = fused ? app.key : nullptr;
    a.new_v = fused ? app.value : nullptr;
    a.slot_mapping = fused ? app.slot_mapping : nullptr;
    a.new_k_stride = app.key_stride;
    a.new_v_stride = app.value_stride;
    // Fixed partitions in the matrix-core kernel: one partition per wave where the table
    // holds at least 2 kWaves partitions. Measured on MI355X at 512-token partitions: the
    // 70B batch 397.5 -> 337.8 us, the 131K-262K-token batch 602-610 -> 573-580 us; the 8B
    // batch (at most 4 partitions per sequence, most sequences in one or two) 63.0 -> 64.4
    // us, so short tables keep the W waves per partition.
    // (32-token blocks in partitions of whole blocks take the whole-block kernel instead)
    a.per_wave = !split && grid_parts >= 2 * pkv::kWaves && in_dtype != PKV_F32 &&
                 !(block_size == 32 && part_tiles % 2 == 0);
    const int grid_slots = a.per_wave ? (grid_parts + pkv::kWaves - 1) / pkv::kWaves : grid_parts;
    a.heads_fastest = grid_slots < 8;
    a.lpt_round = 0;
    a.use_order = 0;
    if (!split && grid_parts == 1 && num_seqs <= pkv::kLptMaxSeqs && in_dtype != PKV_F32) {
        if (seq_order) {
            a.use_order = 1;
            for (int32_t i = 0; i < num_seqs; ++i) a.order[i] = uint16_t(seq_order[i]);
        } else {
            a.lpt_round = std::max(1, pkv::device_cus() / num_kv_heads);
        }
    }
    const dim3 grid = a.heads_fastest
                          ? dim3{unsigned(num_kv_heads), unsigned(num_seqs), unsigned(grid_slots)}
                          : dim3{unsigned(grid_slots), unsigned(num_kv_heads), unsigned(num_seqs)};
    const hipError_t err =
        block_size == 16 ? pkv::dispatch_bs<16>(a, head_dim, in_dtype, out_dtype, grid, s, split, fp8)
        : block_size == 8 ? pkv::dispatch_bs<8>(a, head_dim, in_dtype, out_dtype, grid, s, split, fp8)
                          : pkv::dispatch_bs<32>(a, head_dim, in_dtype, out_dtype, grid, s, split, fp8);
    if (err != hipSuccess)
        return fail(PKV_EHIP, "%s: launch failed: %s", who, hipGetErrorString(err));
    return pkv::ok();
}

}  // namespace

extern "C" int paged_attention_decode(void* out, float* part_out, float* part_max,
                                      float* part_sum, const void* q, int64_t q_stride,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                      int32_t partition_size, int32_t max_partitions,
                                      int32_t in_dtype, int32_t out_dtype,
                                      const int32_t* seq_order, void* stream) {
    return decode_impl("paged_attention_decode", out, part_out, part_max, part_sum, q, q_stride,
                       k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                       head_dim, block_size, max_blocks_per_seq, num_blocks, scale, partition_size,
                       max_partitions, in_dtype, out_dtype, in_dtype, 1.0f, 1.0f,
                       AppendIn{nullptr, nullptr, 0, 0, nullptr}, seq_order, stream);
}

extern "C" int paged_attention_decode_append(
    void* out, float* part_out, float* part_max, float* part_sum, const void* q, int64_t q_stride,
    const void* key, const void* value, int64_t key_stride, int64_t value_stride,
    const int32_t* slot_mapping, void* k_cache, void* v_cache, const int32_t* block_tables,
    const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
    float scale, int32_t partition_size, int32_t max_partitions, int32_t in_dtype,
    int32_t out_dtype, const int32_t* seq_order, void* stream) {
    if (num_seqs > 0 && !key)
        return pkv::fail(PKV_EINVAL, "paged_attention_decode_append: NULL key");
    return decode_impl("paged_attention_decode_append", out, part_out, part_max, part_sum, q,
                       q_stride, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                       partition_size, max_partitions, in_dtype, out_dtype, in_dtype, 1.0f, 1.0f,
                       AppendIn{key, value, key_stride, value_stride, slot_mapping}, seq_order,
                       stream);
}

extern "C" int paged_attention_decode_fp8(void* out, float* part_out, float* part_max,
                                          float* part_sum, const void* q, int64_t q_stride,
                                          const void* k_cache, const void* v_cache,
                                          const int32_t* block_tables, const int32_t* seq_lens,
                                          int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_blocks_per_seq,
                                          int64_t num_blocks, float scale, float k_scale,
                                          float v_scale, int32_t partition_size,
                                          int32_t max_partitions, int32_t in_dtype,
                                          int32_t out_dtype, const int32_t* seq_order,
                                          void* stream) {
    return decode_impl("paged_attention_decode_fp8", out, part_out, part_max, part_sum, q,
                       q_stride, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                       partition_size, max_partitions, in_dtype, out_dtype, PKV_FP8_E4M3, k_scale,
                       v_scale, AppendIn{nullptr, nullptr, 0, 0, nullptr}, seq_order, stream);
}

extern "C" int paged_attention_decode_append_fp8(
    void* out, float* part_out, float* part_max, float* part_sum, const void* q, int64_t q_stride,
    const void* key, const void* value, int64_t key_stride, int64_t value_stride,
    const int32_t* slot_mapping, void* k_cache, void* v_cache, const int32_t* block_tables,
    const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
    float scale, float k_scale, float v_scale, int32_t partition_size, int32_t max_partitions,
    int32_t in_dtype, int32_t out_dtype, const int32_t* seq_order, void* stream) {
    if (num_seqs > 0 && !key)
        return pkv::fail(PKV_EINVAL, "paged_attention_decode_append_fp8: NULL key");
    return decode_impl("paged_attention_decode_append_fp8", out, part_out, part_max, part_sum, q,
                       q_stride, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                       partition_size, max_partitions, in_dtype, out_dtype, PKV_FP8_E4M3, k_scale,
                       v_scale, AppendIn{key, value, key_stride, value_stride, slot_mapping},
                       seq_order, stream);
}

extern "C" int paged_attention_decode_plan(const int32_t* seq_lens, int32_t num_seqs,
                                           int32_t num_kv_heads, int32_t* order_out) {
    using pkv::fail;
    if (num_seqs < 0 || num_kv_heads <= 0)
        return fail(PKV_EINVAL, "paged_attention_decode_plan: bad num_seqs / num_kv_heads");
    if (num_seqs == 0) return pkv::ok();
    if (!seq_lens || !order_out) return fail(PKV_EINVAL, "paged_attention_decode_plan: NULL");
    // rank r = the r-th longest (ties by index); slot b of round r = b / R takes rank
    // R r + pos, or R r + (hi - 1 - pos) in odd rounds
    std::vector<int32_t> by_rank(static_cast<size_t>(num_seqs));
    std::iota(by_rank.begin(), by_rank.end(), 0);
    auto len = [&](int32_t i) { return seq_lens[i] < 0 ? 0 : seq_lens[i]; };
    std::stable_sort(by_rank.begin(), by_rank.end(),
                     [&](int32_t x, int32_t y) { return len(x) > len(y); });
    const int32_t R = std::max(1, pkv::device_cus() / num_kv_heads);
    for (int32_t b = 0; b < num_seqs; ++b) {
        const int32_t r = b / R, pos = b - r * R, hi = std::min(R, num_seqs - r * R);
        order_out[b] = by_rank[size_t(r * R + ((r & 1) ? hi - 1 - pos : pos))];
    }
    return pkv::ok();
}

// ---- decode without allocation -----------------------------------------------------
// paged_attention_decode_noalloc: a partitioned decode and its reduce in one call, for
// callers that cannot allocate device memory. The partition records (part_out, part_max,
// part_sum) live in `scratch`, a file-scope device array that the runtime reserves on each
// device when this code object is first used there and keeps until the process ends. Every
// call on a device shares that device's array: calls that overlap on one device (two
// streams, two threads) race on it. Nothing in it has to start at zero: the decode writes
// every record the reduce reads, so the contents a previous call left do not matter.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up on the first call made
// with that device current and kept. In host code the name `scratch` stands for a
// host-side shadow, not device memory: only this address may reach a kernel.
int scratch_address(const char* who, char** out) {
    static std::mutex mu;
    static void* addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return pkv::fail(PKV_EHIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return pkv::fail(PKV_ENOTSUP, "%s: device ordinal %d", who, dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return pkv::fail(PKV_EHIP, "%s: hipGetSymbolAddress(scratch): %s", who,
                             hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = static_cast<char*>(addr[dev]);
    return PKV_OK;
}

size_t round_up_256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

extern "C" size_t paged_attention_decode_noalloc_workspace(void) { return kScratchBytes; }

extern "C" int paged_attention_decode_noalloc(void* out, const void* q, int64_t q_stride,
                                              const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, const int32_t* seq_lens,
                                              int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t block_size, int32_t max_blocks_per_seq,
                                              int64_t num_blocks, float scale,
                                              int32_t partition_size, int32_t in_dtype,
                                              int32_t out_dtype, void* stream) {
    using pkv::fail;
    const char* who = "paged_attention_decode_noalloc";
    const AppendIn none{nullptr, nullptr, 0, 0, nullptr};
    if (partition_size == 0)   // the single pass keeps no records
        return decode_impl(who, out, nullptr, nullptr, nullptr, q, q_stride, k_cache, v_cache,
                           block_tables, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                           block_size, max_blocks_per_seq, num_blocks, scale, 0, 0, in_dtype,
                           out_dtype, in_dtype, 1.0f, 1.0f, none, nullptr, stream);
    // Sizes of the records, from arguments decode_impl checks again below.
    if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
        (block_size != 8 && block_size != 16 && block_size != 32) ||
        int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
        return fail(PKV_EINVAL, "%s: bad num_seqs / num_heads / head_dim / block_size / "
                                "max_blocks_per_seq", who);
    if (partition_size != PKV_PARTITION_AUTO && (partition_size < 0 || partition_size % 16))
        return fail(PKV_EINVAL, "%s: partition_size must be 0, PKV_PARTITION_AUTO or a "
                                "positive multiple of 16", who);
    const int64_t max_tiles = (int64_t(max_blocks_per_seq) * block_size + 15) / 16;
    const int64_t rows = int64_t(num_seqs) * num_heads;   // (b, h) rows of records
    const int64_t rec_bytes = (int64_t(head_dim) + 2) * 4;  // o, m and l of one record
    int64_t maxp;
    if (partition_size == PKV_PARTITION_AUTO) {
        // The bound paged_attention_decode's callers use (pieces of at least four tiles),
        // lowered to what the workspace holds: fewer records per row only make the pieces
        // longer (the split stays balanced up to that length).
        maxp = std::max<int64_t>(2, (max_tiles + 3) / 4 + 1);
        const int64_t fit = rows > 0 ? int64_t(kScratchBytes - 512) / (rows * rec_bytes) : maxp;
        maxp = std::min(maxp, fit);
        if (maxp < 2)
            return fail(PKV_EINVAL, "%s: %lld (sequence, head) rows need %lld bytes of workspace "
                                    "for two records each, above the %zu-byte static workspace",
                        who, (long long)rows, (long long)(2 * rows * rec_bytes), kScratchBytes);
    } else {
        maxp = (max_tiles + partition_size / 16 - 1) / (partition_size / 16);
        if (rows * maxp * rec_bytes + 512 > int64_t(kScratchBytes))
            return fail(PKV_EINVAL, "%s: %lld rows x %lld partitions need %lld bytes of workspace, "
                                    "above the %zu-byte static workspace (use larger partitions or "
                                    "paged_attention_decode with caller-owned buffers)",
                        who, (long long)rows, (long long)maxp,
                        (long long)(rows * maxp * rec_bytes), kScratchBytes);
    }
    if (maxp > INT32_MAX) return fail(PKV_EINVAL, "%s: too many partitions", who);
    if (num_seqs > 0 && (!out || (reinterpret_cast<uintptr_t>(out) & 15)))
        return fail(PKV_EINVAL, "%s: out must be non-NULL and 16-byte aligned", who);
    char* ws = nullptr;
    if (num_seqs > 0) {
        const int rc = scratch_address(who, &ws);
        if (rc != PKV_OK) return rc;
    }
    // part_out [rows][maxp][d], then part_max and part_sum [rows][maxp], 256-byte aligned
    const size_t o_bytes = round_up_256(size_t(rows * maxp * head_dim) * 4);
    const size_t m_bytes = round_up_256(size_t(rows * maxp) * 4);
    float* part_out = reinterpret_cast<float*>(ws);
    float* part_max = reinterpret_cast<float*>(ws + o_bytes);
    float* part_sum = reinterpret_cast<float*>(ws + o_bytes + m_bytes);
    int rc = decode_impl(who, out, part_out, part_max, part_sum, q, q_stride, k_cache, v_cache,
                         block_tables, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                         block_size, max_blocks_per_seq, num_blocks, scale, partition_size,
                         int32_t(maxp), in_dtype, out_dtype, in_dtype, 1.0f, 1.0f, none, nullptr,
                         stream);
    if (rc != PKV_OK || num_seqs == 0) return rc;
    return paged_attention_reduce(out, part_out, part_max, part_sum, seq_lens, num_seqs, num_heads,
                                  num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                  partition_size, int32_t(maxp), out_dtype, stream);
}
