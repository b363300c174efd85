// paged_attention_reduce: merge the per-partition results of a long context.
//
// Each partition p of a sequence carries o_p (attention restricted to its tokens),
// m_p (its largest logit) and l_p (sum of exp(s - m_p)); the full result is
// sum_p w_p o_p / sum_p w_p with w_p = exp(m_p - max_q m_q) l_p. This is the same
// softmax, evaluated piecewise: the attention math itself is unchanged
// ("vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem, closing paragraphs).
//
// One workgroup of W waves per (query head, sequence): wave w takes partitions
// w, w + W, ...; lane l owns head_dim / 64 consecutive dimensions; the waves'
// partial sums meet in LDS.
#include <hip/hip_runtime.h>

#include <cmath>

#include "device.hpp"
#include "status.hpp"

namespace pkv {

struct ReduceArgs {
    void* out;
    const float* part_out;
    const float* part_max;
    const float* part_sum;
    const int32_t* seq_lens;
    int32_t num_heads;
    int32_t part_tokens;
    int32_t max_partitions;
};

constexpr float kLog2eR = 1.44269504088896340736f;

template <int D, typename OutT, int W>
__global__ __launch_bounds__(W * 64) void reduce_kernel(ReduceArgs a) {
    constexpr int PER = D / 64;   // dimensions per lane
    __shared__ float sm_acc[W][D];
    __shared__ float sm_w[W];
    __shared__ float sm_max[W];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.x, b = blockIdx.y;
    const int n = a.seq_lens[b];
    if (n <= a.part_tokens) return;   // one partition (or none): decode wrote out
    int np = (n + a.part_tokens - 1) / a.part_tokens;
    np = np > a.max_partitions ? a.max_partitions : np;
    const int64_t row = (int64_t(b) * a.num_heads + h) * a.max_partitions;
    const float* pm = a.part_max + row;
    const float* ps = a.part_sum + row;

    // global max of the partition maxima
    float M = -INFINITY;
    for (int p = threadIdx.x; p < np; p += W * 64) M = fmaxf(M, pm[p]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, __shfl_xor(M, s, 64));
    if (lane == 0) sm_max[wave] = M;
    __syncthreads();
    M = sm_max[0];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, sm_max[w]);

    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    float wsum = 0.f;
    for (int p = wave; p < np; p += W) {
        const float wp = exp2_fast((pm[p] - M) * kLog2eR) * ps[p];
        wsum += wp;
        const float* o = a.part_out + (row + p) * D + lane * PER;
        if constexpr (PER == 2) {
            const float2 v = *reinterpret_cast<const float2*>(o);
            acc[0] += wp * v.x;
            acc[1] += wp * v.y;
        } else {
#pragma unroll
            for (int k = 0; k < PER; ++k) acc[k] += wp * o[k];
        }
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) sm_acc[wave][lane * PER + k] = acc[k];
    if (lane == 0) sm_w[wave] = wsum;
    __syncthreads();
    if (wave == 0) {
        float W_ = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) W_ += sm_w[w];
        const float inv = 1.f / W_;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) s += sm_acc[w][lane * PER + k];
            OutStore<OutT>::st(a.out, (int64_t(b) * a.num_heads + h) * D + lane * PER + k, s * inv);
        }
    }
}

constexpr int kReduceWaves = 4;

template <int D>
hipError_t dispatch_reduce(const ReduceArgs& a, int out_dtype, dim3 grid, hipStream_t s) {
    const dim3 block(kReduceWaves * 64);
    if (out_dtype == PKV_F32)
        hipLaunchKernelGGL((reduce_kernel<D, float, kReduceWaves>), grid, block, 0, s, a);
    else if (out_dtype == PKV_BF16)
        hipLaunchKernelGGL((reduce_kernel<D, bf16_t, kReduceWaves>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((reduce_kernel<D, f16_t, kReduceWaves>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace pkv

extern "C" int paged_attention_reduce(void* out, const float* part_out, const float* part_max,
                                      const float* part_sum, const int32_t* seq_lens,
                                      int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                      int32_t partition_size, int32_t max_partitions,
                                      int32_t out_dtype, void* stream) {
    using pkv::fail;
    if (pkv::elem_bytes(out_dtype) == 0)
        return fail(PKV_EINVAL, "paged_attention_reduce: unknown out_dtype %d", out_dtype);
    if (num_seqs < 0 || num_heads <= 0 || num_seqs > 65535)
        return fail(PKV_EINVAL, "paged_attention_reduce: bad num_seqs / num_heads");
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_ENOTSUP, "paged_attention_reduce: head_dim %d (built: 64, 128)", head_dim);
    if (partition_size <= 0 || partition_size % PKV_BLOCK_SIZE || max_partitions <= 0)
        return fail(PKV_EINVAL, "paged_attention_reduce: bad partition_size / max_partitions");
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
    a.num_heads = num_heads;
    a.part_tokens = partition_size;
    a.max_partitions = max_partitions;
    const dim3 grid{unsigned(num_heads), unsigned(num_seqs), 1u};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = head_dim == 128 ? pkv::dispatch_reduce<128>(a, out_dtype, grid, s)
                                           : pkv::dispatch_reduce<64>(a, out_dtype, grid, s);
    if (err != hipSuccess)
        return fail(PKV_EHIP, "paged_attention_reduce: launch failed: %s", hipGetErrorString(err));
    return pkv::ok();
}
