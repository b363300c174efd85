// Measuring aids (not steps of the method): what this GPU streams with no indirection,
// and what it gathers of the decode's own K/V tiles through the block tables with no
// arithmetic. The decode kernel's rate is reported against both, and their ratio is the
// cost of reading through the block table that the pages ask to be counted ("vLLM ve
// Triton ile maliyet optimizasyonu", §05 Sınırlar, on the kernel complexity and
// indirection cost of paged reads).
//
// Every loaded 16-byte group is folded into a running XOR that each wave stores to its own
// slot of `sink` (wave index modulo sink_len), so no load can be dropped and, with a sink of
// at least one slot per wave that starts at zero, the XOR over the sink is the XOR of
// every 32-bit word read; nothing else is written. Each kernel runs with plain or
// non-temporal loads (the decode kernels use the latter for their tiles).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device.hpp"
#include "split.hpp"
#include "status.hpp"
#include "timer.hpp"

namespace pkv {

int device_cus();   // decode.hip

namespace {

__device__ __forceinline__ uint32_t fold(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4* p) {
    if constexpr (NT) return ld_once16(p);
    else return *p;
}

// Contiguous read of n16 16-byte groups: each wave reads U consecutive 1 KiB chunks (one
// 16-byte group per lane and chunk) per round, U loads in flight per lane.
template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                           uint32_t* sink, int32_t sink_len) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
    uint32_t acc = 0;
    for (int64_t c0 = wave * U; c0 * 64 < n16; c0 += waves * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = (c0 + u) * 64 + lane;
            v[u] = i < n16 ? ld16<NT>(buf + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if (lane == 0) sink[(int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6)) % sink_len] = acc;
}

struct GatherArgs {
    const char* k_cache;
    const char* v_cache;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    int64_t num_blocks;
    int64_t tile_bytes;      // one (block, KV head) tile of K (or V): contiguous
    int32_t num_kv_heads;
    int32_t num_seqs;
    int32_t max_blocks;
    int32_t block_size;
    int32_t max_len;
    uint32_t* sink;
    int32_t sink_len;
    SplitParams split;
    int32_t use_order;
    uint16_t order[256];
};

// Load the K and V tile of block id `blk` (KV head g): NL 16-byte groups per lane each.
template <int NL>
struct Tile {
    uint4 k[NL], v[NL];
};
// As the decode kernels read their tiles: through a buffer resource per tile, each lane at
// a fixed offset (see tile_rsrc), so the loop's address registers do not change.
template <bool NT, int NL>
__device__ __forceinline__ void load_tile(Tile<NL>& t, const GatherArgs& a, int blk, int g,
                                          int lane) {
    const bool ok = uint32_t(blk) < block_limit(a.num_blocks);   // an invalid id reads block 0
    const int64_t off = (int64_t(ok ? blk : 0) * a.num_kv_heads + g) * a.tile_bytes;
    const buf_rsrc_t kr = tile_rsrc(a.k_cache + off, int(a.tile_bytes));
    const buf_rsrc_t vr = tile_rsrc(a.v_cache + off, int(a.tile_bytes));
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const u32x4_t k = __builtin_amdgcn_raw_buffer_load_b128(kr, (64 * i + lane) * 16, 0, NT ? kBufNT : 0);
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(vr, (64 * i + lane) * 16, 0, NT ? kBufNT : 0);
        t.k[i] = make_uint4(k[0], k[1], k[2], k[3]);
        t.v[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}
template <int NL>
__device__ __forceinline__ uint32_t fold_tile(const Tile<NL>& t) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < NL; ++i) x ^= fold(t.k[i]) ^ fold(t.v[i]);
    return x;
}

// The single pass's decomposition: one workgroup of 4 waves per (KV head, sequence) in the
// decode's grid order (KV heads fastest, sequences in the host plan's order); the waves
// take the sequence's blocks round-robin, block ids read 64 at a time (one per lane), two
// tiles in flight per wave.
template <int NL, bool NT>
__global__ __launch_bounds__(256) void gather_seq_kernel(GatherArgs a) {
    constexpr int W = 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = blockIdx.x;
    int b = blockIdx.y;
    if (a.use_order) b = a.order[b];
    const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;
    int n = a.seq_lens[b];
    n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
    const int nblk = (n + a.block_size - 1) / a.block_size;
    const int nmine = wave < nblk ? (nblk - wave + W - 1) / W : 0;
    uint32_t acc = 0;
    for (int k0 = 0; k0 < nmine; k0 += 64) {
        const int cnt = min(64, nmine - k0);
        const int j = wave + (k0 + lane) * W;
        const int id = lane < cnt ? table[j] : -1;
        Tile<NL> X, Y;
        load_tile<NT>(X, a, __builtin_amdgcn_readlane(id, 0), g, lane);
        for (int k = 0; k < cnt; k += 2) {
            load_tile<NT>(Y, a, __builtin_amdgcn_readlane(id, min(k + 1, cnt - 1)), g, lane);
            acc ^= fold_tile(X);
            if (k + 1 >= cnt) break;
            load_tile<NT>(X, a, __builtin_amdgcn_readlane(id, min(k + 2, cnt - 1)), g, lane);
            acc ^= fold_tile(Y);
        }
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if (lane == 0) a.sink[((int64_t(blockIdx.y) * gridDim.x + blockIdx.x) * W + wave) % a.sink_len] = acc;
}

// Perfect balance: every (sequence, KV head, block) tile of the batch in one list (order
// b, g, j), cut into equal runs, one per wave (the balanced split's plan, 16-token blocks).
template <int NL, bool NT>
__global__ __launch_bounds__(kSplitThreads) void gather_balanced_kernel(GatherArgs a) {
    __shared__ int32_t s_end[kSplitMaxSeqs];
    __shared__ int32_t s_len[kSplitMaxSeqs];
    __shared__ int32_t s_wave[kSplitThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hkv = a.num_kv_heads;
    const int total = split_scan(a.seq_lens, a.num_seqs, hkv, a.max_len, s_end, s_len, s_wave);
    const int share = split_share(total, a.split);
    const int u = blockIdx.x * (kSplitThreads / 64) + wave;
    const int64_t t0l = int64_t(u) * share;
    uint32_t acc = 0;
    if (t0l < total) {
        const int t1 = min(total, int(t0l) + share);
        for (int tb = int(t0l); tb < t1; tb += 64) {
            const int cnt = min(64, t1 - tb);
            int id = -1, lg = 0;
            if (lane < cnt) {
                const int t = tb + lane;
                int lo = 0, hi = a.num_seqs - 1;   // first b with s_end[b] > t
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (s_end[mid] > t) hi = mid; else lo = mid + 1;
                }
                const int nb = (s_len[lo] + 15) >> 4;
                const int r = t - (lo ? s_end[lo - 1] : 0);
                lg = r / nb;
                const int j = r - lg * nb;
                id = j < a.max_blocks ? a.block_tables[int64_t(lo) * a.max_blocks + j] : -1;
            }
            Tile<NL> X, Y;
            load_tile<NT>(X, a, __builtin_amdgcn_readlane(id, 0), __builtin_amdgcn_readlane(lg, 0), lane);
            for (int k = 0; k < cnt; k += 2) {
                const int k1 = min(k + 1, cnt - 1);
                load_tile<NT>(Y, a, __builtin_amdgcn_readlane(id, k1), __builtin_amdgcn_readlane(lg, k1), lane);
                acc ^= fold_tile(X);
                if (k + 1 >= cnt) break;
                const int k2 = min(k + 2, cnt - 1);
                load_tile<NT>(X, a, __builtin_amdgcn_readlane(id, k2), __builtin_amdgcn_readlane(lg, k2), lane);
                acc ^= fold_tile(Y);
            }
        }
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if (lane == 0) a.sink[(int64_t(blockIdx.x) * (kSplitThreads / 64) + wave) % a.sink_len] = acc;
}

template <int NL, bool NT>
hipError_t launch_gather(const GatherArgs& a, bool balanced, hipStream_t s) {
    const LaunchEvents ev = timer_events(PKV_TIMER_MEASURE);
    if (balanced) {
        const int groups = (a.split.units + kSplitThreads / 64 - 1) / (kSplitThreads / 64);
        hipExtLaunchKernelGGL((gather_balanced_kernel<NL, NT>), dim3(groups), dim3(kSplitThreads), 0, s,
                              ev.start, ev.stop, 0, a);
    } else {
        hipExtLaunchKernelGGL((gather_seq_kernel<NL, NT>),
                              dim3(unsigned(a.num_kv_heads), unsigned(a.num_seqs)), dim3(256), 0, s,
                              ev.start, ev.stop, 0, a);
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace pkv

namespace pkv {
namespace {
template <bool NT>
void launch_read(int loads_in_flight, dim3 grid, hipStream_t s, const LaunchEvents& ev,
                 const uint4* b, int64_t n16, uint32_t* sink, int32_t sink_len) {
    switch (loads_in_flight) {
        case 2: hipExtLaunchKernelGGL((stream_read_kernel<2, NT>), grid, dim3(256), 0, s, ev.start, ev.stop, 0, b, n16, sink, sink_len); break;
        case 4: hipExtLaunchKernelGGL((stream_read_kernel<4, NT>), grid, dim3(256), 0, s, ev.start, ev.stop, 0, b, n16, sink, sink_len); break;
        case 8: hipExtLaunchKernelGGL((stream_read_kernel<8, NT>), grid, dim3(256), 0, s, ev.start, ev.stop, 0, b, n16, sink, sink_len); break;
        default: hipExtLaunchKernelGGL((stream_read_kernel<16, NT>), grid, dim3(256), 0, s, ev.start, ev.stop, 0, b, n16, sink, sink_len); break;
    }
}
// ---- unit rates: what one CU's SIMDs sustain on the operations the kernels are made of
// (LDS operand reads, exponentials, FMAs, 16x16x32 bf16 matrix products, and products mixed
// in one wave with exponentials or FMAs that do not depend on them), at a chosen number of
// waves per SIMD. Each lane folds its results into the wave's sink slot.
constexpr int kRateLdsChunks = 1024;   // 16 KiB of LDS per workgroup: 8 fit on a CU

__device__ __forceinline__ void rate_sink(uint32_t x, uint32_t* sink, int32_t sink_len) {
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
    if ((threadIdx.x & 63) == 0)
        sink[(int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6)) % sink_len] = x;
}

// Workgroup-local LDS chunk i holds (i, 3i, 5i, 7i); iteration t, read j of thread tid reads
// chunk ((8t + j) * 257 + tid) mod 1024: 8 conflict-free 16-byte reads per lane in flight
// (a wave's 64 lanes read 1 KiB of consecutive chunks, wrapping at the array's end).
__global__ __launch_bounds__(256) void rate_lds_kernel(int32_t iters, uint32_t* sink, int32_t sink_len) {
    __shared__ uint4 buf[kRateLdsChunks];
    const int tid = threadIdx.x;
    for (int i = tid; i < kRateLdsChunks; i += 256) buf[i] = make_uint4(i, 3 * i, 5 * i, 7 * i);
    __syncthreads();
    uint32_t x = 0;
    for (int t = 0; t < iters; ++t) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x ^= fold(buf[((t * 8 + j) * 257 + tid) & (kRateLdsChunks - 1)]);
    }
    rate_sink(x, sink, sink_len);
}

// Per iteration and lane: kind 1: 8 exponentials (independent chains); 2: 8 FMAs; 3: 4
// products (4 accumulator chains); 4: 4 products and 8 exponentials; 5: 4 products and 16
// FMAs, the vector instructions placed between the products; 6: 4 products of the
// 16x16x16 bf16 form (half the work of kind 3's per instruction).
template <int KIND>
__global__ __launch_bounds__(256) void rate_alu_kernel(int32_t iters, uint32_t* sink, int32_t sink_len) {
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    bf16x8_t a, b;
    for (int k = 0; k < 8; ++k) {
        a[k] = (__bf16)(threadIdx.x * 1e-3f);
        b[k] = (__bf16)(k * 1e-2f);
    }
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = threadIdx.x * 1e-3f + k;
    for (int t = 0; t < iters; ++t) {
        if constexpr (KIND == 1 || KIND == 4) {
            if constexpr (KIND == 4) c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
            y[0] = __builtin_amdgcn_exp2f(y[0]);
            y[1] = __builtin_amdgcn_exp2f(y[1]);
            if constexpr (KIND == 4) c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
            y[2] = __builtin_amdgcn_exp2f(y[2]);
            y[3] = __builtin_amdgcn_exp2f(y[3]);
            if constexpr (KIND == 4) c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
            y[4] = __builtin_amdgcn_exp2f(y[4]);
            y[5] = __builtin_amdgcn_exp2f(y[5]);
            if constexpr (KIND == 4) c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
            y[6] = __builtin_amdgcn_exp2f(y[6]);
            y[7] = __builtin_amdgcn_exp2f(y[7]);
        } else if constexpr (KIND == 2 || KIND == 5) {
            if constexpr (KIND == 5) c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = __builtin_fmaf(y[k], 0.999f, 1e-3f);
            if constexpr (KIND == 5) c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
#pragma unroll
            for (int k = 4; k < 8; ++k) y[k] = __builtin_fmaf(y[k], 0.999f, 1e-3f);
            if constexpr (KIND == 5) {
                c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
#pragma unroll
                for (int k = 0; k < 4; ++k) y[k] = __builtin_fmaf(y[k], 0.999f, 1e-3f);
                c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
#pragma unroll
                for (int k = 4; k < 8; ++k) y[k] = __builtin_fmaf(y[k], 0.999f, 1e-3f);
            }
        } else if constexpr (KIND == 6) {
            typedef short i16x4_t __attribute__((ext_vector_type(4)));
            const i16x4_t a4 = __builtin_bit_cast(i16x4_t, a.lo), b4 = __builtin_bit_cast(i16x4_t, b.lo);
            c0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, c3, 0, 0, 0);
        } else {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
        }
    }
    const f32x4 c = (c0 + c1) + (c2 + c3);
    float acc = (c[0] + c[1]) + (c[2] + c[3]);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += y[k];
    rate_sink(__builtin_bit_cast(uint32_t, acc), sink, sink_len);
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_measure_read(const void* buf, int64_t bytes, int32_t waves_per_cu,
                                int32_t loads_in_flight, int32_t nontemporal, uint32_t* sink,
                                int32_t sink_len, void* stream) {
    using pkv::fail;
    const char* who = "pkv_measure_read";
    if (!buf || !sink || sink_len <= 0 || bytes < 0 || (bytes & 15) ||
        (reinterpret_cast<uintptr_t>(buf) & 15))
        return fail(PKV_EINVAL, "%s: NULL, misaligned or bad size", who);
    if (waves_per_cu < 4 || waves_per_cu > 32 || waves_per_cu % 4)
        return fail(PKV_EINVAL, "%s: waves_per_cu must be 4 .. 32, a multiple of 4", who);
    if (loads_in_flight != 2 && loads_in_flight != 4 && loads_in_flight != 8 &&
        loads_in_flight != 16)
        return fail(PKV_EINVAL, "%s: loads_in_flight must be 2, 4, 8 or 16", who);
    if (bytes == 0) return pkv::ok();
    const dim3 grid(unsigned(pkv::device_cus() * waves_per_cu / 4));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const pkv::LaunchEvents ev = pkv::timer_events(PKV_TIMER_MEASURE);
    const uint4* b = static_cast<const uint4*>(buf);
    const int64_t n16 = bytes / 16;
    if (nontemporal)
        pkv::launch_read<true>(loads_in_flight, grid, s, ev, b, n16, sink, sink_len);
    else
        pkv::launch_read<false>(loads_in_flight, grid, s, ev, b, n16, sink, sink_len);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(PKV_EHIP, "%s: launch failed: %s", who, hipGetErrorString(err));
    return pkv::ok();
}

extern "C" int pkv_measure_gather(const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t cache_dtype,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  const int32_t* seq_order, int32_t balanced, int32_t nontemporal,
                                  uint32_t* sink, int32_t sink_len, void* stream) {
    using pkv::fail;
    const char* who = "pkv_measure_gather";
    const int e = pkv::cache_elem_bytes(cache_dtype);
    if (e == 0) return fail(PKV_EINVAL, "%s: unknown cache dtype %d", who, cache_dtype);
    if (num_seqs < 0 || num_seqs > 65535 || num_kv_heads <= 0 || num_kv_heads > 65535 ||
        head_dim <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || sink_len <= 0 ||
        int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
        return fail(PKV_EINVAL, "%s: bad sizes", who);
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PKV_EINVAL, "%s: block_size must be 8, 16 or 32", who);
    if (balanced && (block_size != 16 || num_seqs > pkv::kSplitMaxSeqs))
        return fail(PKV_ENOTSUP, "%s: the balanced gather takes 16-token blocks and at most %d "
                                 "sequences", who, pkv::kSplitMaxSeqs);
    const int64_t tile_bytes = int64_t(head_dim) * block_size * e;
    const int nl = int(tile_bytes / 1024);
    if (tile_bytes % 1024 || (nl != 1 && nl != 2 && nl != 4 && nl != 8))
        return fail(PKV_ENOTSUP, "%s: tiles of %lld bytes (built: 1, 2, 4 or 8 KiB)", who,
                    (long long)tile_bytes);
    if (num_seqs == 0) return pkv::ok();
    if (!k_cache || !v_cache || !block_tables || !seq_lens || !sink)
        return fail(PKV_EINVAL, "%s: NULL pointer", who);
    if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
        return fail(PKV_EINVAL, "%s: caches must be 16-byte aligned", who);
    pkv::GatherArgs a;
    a.k_cache = static_cast<const char*>(k_cache);
    a.v_cache = static_cast<const char*>(v_cache);
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.num_blocks = num_blocks;
    a.tile_bytes = tile_bytes;
    a.num_kv_heads = num_kv_heads;
    a.num_seqs = num_seqs;
    a.max_blocks = max_blocks_per_seq;
    a.block_size = block_size;
    a.max_len = max_blocks_per_seq * block_size;
    a.sink = sink;
    a.sink_len = sink_len;
    a.split.units = pkv::device_cus() * 8;   // the balanced split's 8 waves per CU
    a.split.min_share = 1;
    a.use_order = 0;
    if (seq_order && !balanced && num_seqs <= 256) {
        a.use_order = 1;
        for (int32_t i = 0; i < num_seqs; ++i) {
            if (seq_order[i] < 0 || seq_order[i] >= num_seqs)
                return fail(PKV_EINVAL, "%s: seq_order out of range", who);
            a.order[i] = uint16_t(seq_order[i]);
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    const bool bal = balanced != 0;
    if (nontemporal) {
        switch (nl) {
            case 1: err = pkv::launch_gather<1, true>(a, bal, s); break;
            case 2: err = pkv::launch_gather<2, true>(a, bal, s); break;
            case 4: err = pkv::launch_gather<4, true>(a, bal, s); break;
            default: err = pkv::launch_gather<8, true>(a, bal, s); break;
        }
    } else {
        switch (nl) {
            case 1: err = pkv::launch_gather<1, false>(a, bal, s); break;
            case 2: err = pkv::launch_gather<2, false>(a, bal, s); break;
            case 4: err = pkv::launch_gather<4, false>(a, bal, s); break;
            default: err = pkv::launch_gather<8, false>(a, bal, s); break;
        }
    }
    if (err != hipSuccess) return fail(PKV_EHIP, "%s: launch failed: %s", who, hipGetErrorString(err));
    return pkv::ok();
}

extern "C" int pkv_measure_rate(int32_t kind, int32_t waves_per_simd, int32_t iters,
                                uint32_t* sink, int32_t sink_len, void* stream) {
    using pkv::fail;
    const char* who = "pkv_measure_rate";
    if (!sink || sink_len <= 0 || iters < 0)
        return fail(PKV_EINVAL, "%s: NULL sink, bad sink_len or negative iters", who);
    if (kind < 0 || kind > 6) return fail(PKV_EINVAL, "%s: kind must be 0 .. 6", who);
    if (waves_per_simd < 1 || waves_per_simd > 8)
        return fail(PKV_EINVAL, "%s: waves_per_simd must be 1 .. 8", who);
    // workgroups of 4 waves, one per SIMD of a CU: waves_per_simd workgroups per CU
    const dim3 grid(unsigned(pkv::device_cus() * waves_per_simd));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const pkv::LaunchEvents ev = pkv::timer_events(PKV_TIMER_MEASURE);
    switch (kind) {
    case 0: hipExtLaunchKernelGGL(pkv::rate_lds_kernel, grid, dim3(256), 0, s, ev.start, ev.stop, 0, iters, sink, sink_len); break;
    case 1: hipExtLaunchKernelGGL(pkv::rate_alu_kernel<1>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, iters, sink, sink_len); break;
    case 2: hipExtLaunchKernelGGL(pkv::rate_alu_kernel<2>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, iters, sink, sink_len); break;
    case 3: hipExtLaunchKernelGGL(pkv::rate_alu_kernel<3>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, iters, sink, sink_len); break;
    case 4: hipExtLaunchKernelGGL(pkv::rate_alu_kernel<4>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, iters, sink, sink_len); break;
    case 5: hipExtLaunchKernelGGL(pkv::rate_alu_kernel<5>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, iters, sink, sink_len); break;
    default: hipExtLaunchKernelGGL(pkv::rate_alu_kernel<6>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, iters, sink, sink_len); break;
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(PKV_EHIP, "%s: launch failed: %s", who, hipGetErrorString(err));
    return pkv::ok();
}
