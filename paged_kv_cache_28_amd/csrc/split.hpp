// Balanced split of the decode work (partition_size == PKV_PARTITION_AUTO).
//
// All (sequence b, KV head g, logical block j) tiles, taken in the order b, g, j, form
// one list of T tiles. Wave u of the decode launch takes the contiguous run
// [u * s, (u + 1) * s) with s = max(ceil(T / units), min_share), so every wave streams
// the same number of tiles however ragged the lengths are. The run of one (b, g) that
// falls to one wave is a "piece"; a (b, g) whose tiles all fall to one wave is written
// straight to the output, the others leave one partial record per piece for the
// reduce. Piece k of (b, g) is the one taken by wave floor(start / s) + k, where start
// is the index of the first tile of (b, g). Both kernels derive the same plan from
// the sequence lengths, so nothing else has to pass between them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kSplitMaxSeqs = 1024;   // sequences per launch in the balanced mode
constexpr int kSplitThreads = 256;    // workgroup size of both kernels in that mode

struct SplitParams {
    int32_t units;       // waves of the decode launch
    int32_t min_share;   // lower bound of s: keeps pieces per (b, g) <= max_partitions
};

// Workgroup-wide: s_len[b] = n_b clamped to [0, max_len], s_end[b] = sum over b' <= b
// of hkv * ceil(n_b' / 16). Returns T. All kSplitThreads threads must call it.
__device__ inline int32_t split_scan(const int32_t* __restrict__ seq_lens, int num_seqs, int hkv,
                                     int max_len, int32_t* s_end, int32_t* s_len, int32_t* s_wave) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kWavesPerGroup = kSplitThreads / 64;
    const int per = (num_seqs + kSplitThreads - 1) / kSplitThreads;
    const int lo = tid * per, hi = min(num_seqs, lo + per);
    int local = 0;
    for (int b = lo; b < hi; ++b) {
        int n = seq_lens[b];
        n = n < 0 ? 0 : (n > max_len ? max_len : n);
        s_len[b] = n;
        local += hkv * ((n + 15) >> 4);
    }
    int incl = local;   // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
        base += w < wave ? s_wave[w] : 0;
        total += s_wave[w];
    }
    int run = base + incl - local;
    for (int b = lo; b < hi; ++b) {
        run += hkv * ((s_len[b] + 15) >> 4);
        s_end[b] = run;
    }
    __syncthreads();
    return total;
}

// Host side: waves of a balanced-mode decode launch on the current device (the
// resident capacity: compute units x waves per unit). Both launchers call it, so the
// decode and the reduce of one step agree on the plan.
int split_units();

__device__ inline int32_t split_share(int32_t total, const SplitParams& p) {
    int32_t s = (total + p.units - 1) / p.units;
    s = s < p.min_share ? p.min_share : s;
    return s < 1 ? 1 : s;
}

}  // namespace pkv
