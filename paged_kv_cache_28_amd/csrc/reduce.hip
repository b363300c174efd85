// paged_attention_reduce: merge the per-partition results of a long context.
//
// Each partition p of a sequence carries o_p (attention restricted to its tokens),
// m_p (its largest logit) and l_p (sum of exp(s - m_p)); the full result is
// sum_p w_p o_p / sum_p w_p with w_p = exp(m_p - max_q m_q) l_p. This is the same
// softmax, evaluated piecewise: the attention math itself is unchanged
// ("vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem, closing paragraphs).
//
// Each query head's row is merged in 32-dimension slices, one workgroup per slice; the
// records are folded in online by 32 groups of threads and combined through LDS.
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
    int32_t max_len;        // max_blocks_per_seq * block_size
    int32_t part_tokens;
    int32_t max_partitions;
    SplitParams split;
    int32_t heads_per_wg;   // consecutive heads merged by one workgroup (1 or G)
    int32_t grouped;        // 1: grid (KV head, 1, sequence), heads_per_wg = G
};

constexpr float kLog2eR = 1.44269504088896340736f;

// Row (b, h) is cut into slices of S dimensions. A workgroup takes one slice of hw
// consecutive heads of one sequence: thread t owns the four dimensions 4 (t % (S/4)) .. + 3
// of head t / (S/4) % hw, for the records p = rg (mod RG), rg = t / (hw S/4). It folds
// them in online (running maximum of the reference points), and the RG record groups are
// then combined through LDS. Every record is read once, in one pass, with many records in
// flight per workgroup. Fixed partitions (many records per row) use 32-dimension slices
// of single heads; the balanced split uses whole rows, of single heads when there are
// few (sequence, KV head) pairs, else of all G heads of a KV head, so the plan prefix is
// computed once per (sequence, KV head).
template <int D, typename OutT, bool Split, int S>
__global__ __launch_bounds__(256) void reduce_rows_kernel(ReduceArgs a) {
    constexpr int kDimLanes = S / 4;                // threads per record and head (float4 each)
    __shared__ float s_m[256];
    __shared__ float s_w[256];
    __shared__ float4 s_o[256];
    __shared__ int32_t s_red[2 * 4];
    const int hw = a.heads_per_wg;
    const int per = kDimLanes * hw;                 // threads per record group
    const int RG = 256 / per;                       // record groups
    const int t = threadIdx.x, dl = t % kDimLanes, hh = (t / kDimLanes) % hw, rg = t / per;
    // grouped grid (KV head, 1, sequence): whole rows of heads g*hw ..; otherwise
    // (slice, head, sequence)
    const int slice = a.grouped ? 0 : blockIdx.x;
    const int h = a.grouped ? blockIdx.x * hw + hh : blockIdx.y;
    const int b = blockIdx.z;
    const int dim0 = slice * S + 4 * dl;
    const int hkv = a.num_kv_heads, G = a.num_heads / hkv, g = h / G;
    const int max_len = a.max_len;
    const int64_t out_at = (int64_t(b) * a.num_heads + h) * D + dim0;

    int n = a.seq_lens[b];
    n = n < 0 ? 0 : (n > max_len ? max_len : n);
    int np;
    if constexpr (Split) {
        // the plan of the decode launch: this (b, g)'s first tile and the share s
        int before = 0, total = 0;
        for (int i = t; i < a.num_seqs; i += 256) {
            int m = a.seq_lens[i];
            m = m < 0 ? 0 : (m > max_len ? max_len : m);
            const int tiles = hkv * ((m + 15) >> 4);
            total += tiles;
            before += i < b ? tiles : 0;
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            total += __shfl_xor(total, d, 64);
            before += __shfl_xor(before, d, 64);
        }
        if ((t & 63) == 0) {
            s_red[t >> 6] = total;
            s_red[4 + (t >> 6)] = before;
        }
        __syncthreads();
        total = s_red[0] + s_red[1] + s_red[2] + s_red[3];
        before = s_red[4] + s_red[5] + s_red[6] + s_red[7];
        if (n == 0) {   // empty sequence: no tile, so no piece wrote its row
            if (rg == 0) OutStore<OutT>::st4(a.out, out_at, make_float4(0.f, 0.f, 0.f, 0.f));
            return;
        }
        const int share = split_share(total, a.split);
        const int nblk = (n + 15) >> 4;
        const int start = before + g * nblk;
        np = (start + nblk - 1) / share - start / share + 1;
    } else {
        if (n <= a.part_tokens) return;   // one partition (or none): decode wrote out
        np = (n + a.part_tokens - 1) / a.part_tokens;
    }
    np = np > a.max_partitions ? a.max_partitions : np;
    if (np <= 1) return;

    const int64_t row = (int64_t(b) * a.num_heads + h) * a.max_partitions;
    float m = -INFINITY, w = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int p = rg; p < np; p += RG) {   // rg >= RG (idle threads): no record
        const float mp = a.part_max[row + p] * kLog2eR;   // base-2 units
        const float lp = a.part_sum[row + p];
        const float4 v = *reinterpret_cast<const float4*>(a.part_out + (row + p) * D + dim0);
        const float mn = fmaxf(m, mp);
        const float s1 = m == -INFINITY ? 0.f : exp2_fast(m - mn);
        const float s2 = (mp == -INFINITY ? 0.f : exp2_fast(mp - mn)) * lp;
        o.x = o.x * s1 + s2 * v.x;
        o.y = o.y * s1 + s2 * v.y;
        o.z = o.z * s1 + s2 * v.z;
        o.w = o.w * s1 + s2 * v.w;
        w = w * s1 + s2;
        m = mn;
    }
    s_m[t] = m;
    s_w[t] = w;
    s_o[t] = o;
    __syncthreads();
    if (rg != 0) return;
    float M = -INFINITY;
    for (int r = 0; r < RG; ++r) M = fmaxf(M, s_m[r * per + t]);
    float W = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = 0; r < RG; ++r) {
        const float mr = s_m[r * per + t];
        const float f = mr == -INFINITY ? 0.f : exp2_fast(mr - M);   // groups with no record
        const float4 v = s_o[r * per + t];
        W += f * s_w[r * per + t];
        O.x += f * v.x;
        O.y += f * v.y;
        O.z += f * v.z;
        O.w += f * v.w;
    }
    const float inv = 1.f / W;
    OutStore<OutT>::st4(a.out, out_at, make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv));
}

template <int D, typename OutT>
hipError_t launch_reduce(ReduceArgs a, bool split, hipStream_t s) {
    const LaunchEvents ev = timer_events(PKV_TIMER_REDUCE);
    constexpr int kFixedSlice = 32;
    const int G = a.num_heads / a.num_kv_heads;
    if (split) {
        // whole rows; all G heads of a KV head per workgroup when that fills the device
        const bool grouped = G * (D / 4) <= 256 && int64_t(a.num_seqs) * a.num_kv_heads >= 256;
        a.heads_per_wg = grouped ? G : 1;
        a.grouped = grouped;
        const dim3 grid = grouped ? dim3{unsigned(a.num_kv_heads), 1u, unsigned(a.num_seqs)}
                                  : dim3{1u, unsigned(a.num_heads), unsigned(a.num_seqs)};
        hipExtLaunchKernelGGL((reduce_rows_kernel<D, OutT, true, D>), grid, dim3(256), 0, s,
                              ev.start, ev.stop, 0, a);
    } else {
        a.heads_per_wg = 1;
        a.grouped = 0;
        hipExtLaunchKernelGGL((reduce_rows_kernel<D, OutT, false, kFixedSlice>),
                              dim3(unsigned(D / kFixedSlice), unsigned(a.num_heads),
                                   unsigned(a.num_seqs)),
                              dim3(256), 0, s, ev.start, ev.stop, 0, a);
    }
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
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int32_t partition_size,
                                      int32_t max_partitions, int32_t out_dtype, void* stream) {
    using pkv::fail;
    if (pkv::elem_bytes(out_dtype) == 0)
        return fail(PKV_EINVAL, "paged_attention_reduce: unknown out_dtype %d", out_dtype);
    if (num_seqs < 0 || num_seqs > 65535 || num_heads <= 0 || num_heads > 65535 || num_kv_heads <= 0 ||
        num_heads % num_kv_heads || max_blocks_per_seq <= 0)
        return fail(PKV_EINVAL, "paged_attention_reduce: bad num_seqs / heads / max_blocks");
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PKV_EINVAL, "paged_attention_reduce: block_size must be 8, 16 or 32, got %d",
                    block_size);
    if (int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
        return fail(PKV_EINVAL, "paged_attention_reduce: max_blocks_per_seq too large");
    const int32_t max_len = max_blocks_per_seq * block_size;
    const int32_t max_tiles = (max_len + 15) / 16;   // 16-token tiles, as the decode plans
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_ENOTSUP, "paged_attention_reduce: head_dim %d (built: 64, 128)", head_dim);
    const bool split = partition_size == PKV_PARTITION_AUTO;
    if (split) {
        if (num_seqs > pkv::kSplitMaxSeqs || max_partitions < 2 ||
            int64_t(num_seqs) * num_kv_heads * max_tiles >= (int64_t(1) << 31))
            return fail(PKV_EINVAL, "paged_attention_reduce: arguments do not match a "
                                    "PKV_PARTITION_AUTO decode");
    } else if (partition_size <= 0 || partition_size % 16 || max_partitions <= 0) {
        return fail(PKV_EINVAL, "paged_attention_reduce: bad partition_size / max_partitions");
    }
    if (num_seqs == 0) return pkv::ok();
    if (!out || !part_out || !part_max || !part_sum || !seq_lens)
        return fail(PKV_EINVAL, "paged_attention_reduce: NULL pointer");
    if ((reinterpret_cast<uintptr_t>(part_out) | reinterpret_cast<uintptr_t>(out)) & 15)
        return fail(PKV_EINVAL, "paged_attention_reduce: part_out and out must be 16-byte aligned");
    pkv::ReduceArgs a;
    a.out = out;
    a.part_out = part_out;
    a.part_max = part_max;
    a.part_sum = part_sum;
    a.seq_lens = seq_lens;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_len = max_len;
    a.part_tokens = partition_size;
    a.max_partitions = max_partitions;
    a.split.units = split ? pkv::split_units() : 0;
    a.split.min_share = split ? (max_tiles + max_partitions - 2) / (max_partitions - 1) : 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = head_dim == 128 ? pkv::dispatch_reduce<128>(a, out_dtype, split, s)
                                           : pkv::dispatch_reduce<64>(a, out_dtype, split, s);
    if (err != hipSuccess)
        return fail(PKV_EHIP, "paged_attention_reduce: launch failed: %s", hipGetErrorString(err));
    return pkv::ok();
}
