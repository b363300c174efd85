// paged_attention_reduce: merge the per-partition results of a long context.
//
// Each partition p of a sequence carries o_p (attention restricted to its tokens),
// m_p (its largest logit) and l_p (sum of exp(s - m_p)); the full result is
// sum_p w_p o_p / sum_p w_p with w_p = exp(m_p - max_q m_q) l_p. This is the same
// softmax, evaluated piecewise: the attention math itself is unchanged
// ("vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem, closing paragraphs).
//
// Each query head's row is merged by one wave: lane l owns head_dim / 64
// consecutive dimensions and the partitions are folded in online.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>

#include "device.hpp"
#include "split.hpp"
#include "status.hpp"
#include "timer.hpp"

namespace pkv {

struct ReduceArgs {
    void* out;
    const float* part_out;
    const float* part_max;
    const float* part_sum;
    const int32_t* seq_lens;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t max_blocks;
    int32_t part_tokens;
    int32_t max_partitions;
    SplitParams split;
};

constexpr float kLog2eR = 1.44269504088896340736f;
constexpr int kReduceWaves = kSplitThreads / 64;

// Merge the np partial records of row (b, h) with one wave: lane l owns D / 64
// consecutive dimensions; the records' reference points and sums are read 64 at a
// time, one per lane, and merged online (running maximum of the reference points).
template <int D, typename OutT>
__device__ void merge_row(const ReduceArgs& a, int b, int h, int np) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t(b) * a.num_heads + h) * a.max_partitions;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    float M = -INFINITY, wsum = 0.f;
    for (int p0 = 0; p0 < np; p0 += 64) {
        const int cnt = min(64, np - p0);
        const bool live = lane < cnt;
        const float pm = live ? a.part_max[row + p0 + lane] : -INFINITY;
        const float ps = live ? a.part_sum[row + p0 + lane] : 0.f;
        float mc = pm;
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) mc = fmaxf(mc, __shfl_xor(mc, s, 64));
        const float mn = fmaxf(M, mc);
        const float alpha = exp2_fast((M - mn) * kLog2eR);   // 0 on the first chunk
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] *= alpha;
        wsum *= alpha;
        M = mn;
        const float w = live ? exp2_fast((pm - M) * kLog2eR) * ps : 0.f;
        wsum += w;
        const float* o = a.part_out + (row + p0) * D + lane * PER;
#pragma unroll 8
        for (int k = 0; k < cnt; ++k) {
            const float wk = __builtin_bit_cast(float,
                __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
            if constexpr (PER == 2) {
                const float2 v = *reinterpret_cast<const float2*>(o + int64_t(k) * D);
                acc[0] += wk * v.x;
                acc[1] += wk * v.y;
            } else {
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] += wk * o[int64_t(k) * D + e];
            }
        }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) wsum += __shfl_xor(wsum, s, 64);
    const float inv = 1.f / wsum;
#pragma unroll
    for (int k = 0; k < PER; ++k)
        OutStore<OutT>::st(a.out, (int64_t(b) * a.num_heads + h) * D + lane * PER + k, acc[k] * inv);
}

// Fixed partitions: each wave merges one query head, np = ceil(n / P).
template <int D, typename OutT>
__global__ __launch_bounds__(kSplitThreads) void reduce_kernel(ReduceArgs a) {
    const int h = blockIdx.x * kReduceWaves + (threadIdx.x >> 6), b = blockIdx.y;
    if (h >= a.num_heads) return;
    const int n = a.seq_lens[b];
    if (n <= a.part_tokens) return;   // one partition (or none): decode wrote out
    int np = (n + a.part_tokens - 1) / a.part_tokens;
    np = np > a.max_partitions ? a.max_partitions : np;
    merge_row<D, OutT>(a, b, h, np);
}

// Balanced split: one workgroup per (KV head, sequence); its waves merge the G query
// heads of the group; pieces come from the same plan as the decode launch.
template <int D, typename OutT>
__global__ __launch_bounds__(kSplitThreads) void reduce_split_kernel(ReduceArgs a) {
    __shared__ int32_t s_end[kSplitMaxSeqs];
    __shared__ int32_t s_len[kSplitMaxSeqs];
    __shared__ int32_t s_wave[kReduceWaves];
    const int g = blockIdx.x, b = blockIdx.y;
    const int hkv = a.num_kv_heads, G = a.num_heads / hkv;
    const int total = split_scan(a.seq_lens, a.num_seqs, hkv, a.max_blocks * 16, s_end, s_len, s_wave);
    const int share = split_share(total, a.split);
    const int n = s_len[b];
    if (n == 0) {   // empty sequence: no tile, so no piece wrote its rows
        for (int i = threadIdx.x; i < G * D; i += blockDim.x)
            OutStore<OutT>::st(a.out, (int64_t(b) * a.num_heads + g * G + i / D) * D + i % D, 0.f);
        return;
    }
    const int nblk = (n + 15) >> 4;
    const int start = (b ? s_end[b - 1] : 0) + g * nblk;
    const int np = (start + nblk - 1) / share - start / share + 1;
    if (np <= 1) return;
    for (int hh = threadIdx.x >> 6; hh < G; hh += kReduceWaves) merge_row<D, OutT>(a, b, g * G + hh, np);
}

template <int D, typename OutT>
hipError_t launch_reduce(const ReduceArgs& a, bool split, hipStream_t s) {
    const LaunchEvents ev = timer_events(PKV_TIMER_REDUCE);
    if (split)
        hipExtLaunchKernelGGL((reduce_split_kernel<D, OutT>),
                              dim3(unsigned(a.num_kv_heads), unsigned(a.num_seqs), 1u),
                              dim3(kSplitThreads), 0, s, ev.start, ev.stop, 0, a);
    else
        hipExtLaunchKernelGGL((reduce_kernel<D, OutT>),
                              dim3(unsigned((a.num_heads + kReduceWaves - 1) / kReduceWaves),
                                   unsigned(a.num_seqs), 1u),
                              dim3(kSplitThreads), 0, s, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_reduce(const ReduceArgs& a, int out_dtype, bool split, hipStream_t s) {
    if (out_dtype == PKV_F32) return launch_reduce<D, float>(a, split, s);
    if (out_dtype == PKV_BF16) return launch_reduce<D, bf16_t>(a, split, s);
    return launch_reduce<D, f16_t>(a, split, s);
}

}  // namespace pkv

extern "C" int paged_attention_reduce(void* out, const float* part_out, const float* part_max,
                                      const float* part_sum, const int32_t* seq_lens,
                                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_blocks_per_seq,
                                      int32_t partition_size, int32_t max_partitions,
                                      int32_t out_dtype, void* stream) {
    using pkv::fail;
    if (pkv::elem_bytes(out_dtype) == 0)
        return fail(PKV_EINVAL, "paged_attention_reduce: unknown out_dtype %d", out_dtype);
    if (num_seqs < 0 || num_seqs > 65535 || num_heads <= 0 || num_kv_heads <= 0 ||
        num_heads % num_kv_heads || max_blocks_per_seq <= 0)
        return fail(PKV_EINVAL, "paged_attention_reduce: bad num_seqs / heads / max_blocks");
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_ENOTSUP, "paged_attention_reduce: head_dim %d (built: 64, 128)", head_dim);
    const bool split = partition_size == PKV_PARTITION_AUTO;
    if (split) {
        if (num_seqs > pkv::kSplitMaxSeqs || max_partitions < 2 ||
            int64_t(num_seqs) * num_kv_heads * max_blocks_per_seq >= (int64_t(1) << 31))
            return fail(PKV_EINVAL, "paged_attention_reduce: arguments do not match a "
                                    "PKV_PARTITION_AUTO decode");
    } else if (partition_size <= 0 || partition_size % PKV_BLOCK_SIZE || max_partitions <= 0) {
        return fail(PKV_EINVAL, "paged_attention_reduce: bad partition_size / max_partitions");
    }
    if (num_seqs == 0) return pkv::ok();
    if (!out || !part_out || !part_max || !part_sum || !seq_lens)
        return fail(PKV_EINVAL, "paged_attention_reduce: NULL pointer");
    if (reinterpret_cast<uintptr_t>(part_out) & 7)
        return fail(PKV_EINVAL, "paged_attention_reduce: part_out must be 8-byte aligned");
    pkv::ReduceArgs a;
    a.out = out;
    a.part_out = part_out;
    a.part_max = part_max;
    a.part_sum = part_sum;
    a.seq_lens = seq_lens;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.part_tokens = partition_size;
    a.max_partitions = max_partitions;
    a.split.units = split ? pkv::split_units() : 0;
    a.split.min_share = split ? (max_blocks_per_seq + max_partitions - 2) / (max_partitions - 1) : 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = head_dim == 128 ? pkv::dispatch_reduce<128>(a, out_dtype, split, s)
                                           : pkv::dispatch_reduce<64>(a, out_dtype, split, s);
    if (err != hipSuccess)
        return fail(PKV_EHIP, "paged_attention_reduce: launch failed: %s", hipGetErrorString(err));
    return pkv::ok();
}
