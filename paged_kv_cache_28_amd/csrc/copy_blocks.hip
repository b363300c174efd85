// copy_blocks: the device half of copy-on-write. When a sequence appends to a partly
// filled block that other block tables also reference, the pool moves it to a fresh block
// and reports (old, new); this kernel copies the old block onto the new one in the K and
// the V cache of every layer ("vLLM ve Triton ile maliyet optimizasyonu", §03, paragraph
// on sharing: a shared block stays one copy until a user writes to it, and is copied
// then).
//
// One workgroup per (pair, layer, K or V): a block is one contiguous run of block_bytes
// (all KV heads of the block), copied with 16-byte loads and stores. The layers' cache
// pointers travel as kernel arguments, kCopyLayers per launch.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include "status.hpp"
#include "timer.hpp"

namespace pkv {

constexpr int kCopyLayers = 64;
constexpr int kCopyMaxLayers = 256;

struct CopyArgs {
    char* k[kCopyLayers];
    char* v[kCopyLayers];
    const int32_t* pairs;
    int64_t block_bytes;
    int64_t num_blocks;
};

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
    const int p = blockIdx.x, l = blockIdx.y;
    const int32_t src = a.pairs[2 * p], dst = a.pairs[2 * p + 1];
    if (src < 0 || dst < 0 || src >= a.num_blocks || dst >= a.num_blocks || src == dst) return;
    char* base = blockIdx.z ? a.v[l] : a.k[l];
    const uint4* s = reinterpret_cast<const uint4*>(base + int64_t(src) * a.block_bytes);
    uint4* d = reinterpret_cast<uint4*>(base + int64_t(dst) * a.block_bytes);
    const int64_t n = a.block_bytes / 16;
    for (int64_t i = threadIdx.x; i < n; i += 256) d[i] = s[i];
}

}  // namespace pkv

extern "C" int copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                           const int32_t* pairs, int32_t n_pairs, int64_t block_bytes,
                           int64_t num_blocks, void* stream) {
    using pkv::fail;
    if (num_layers < 1 || num_layers > pkv::kCopyMaxLayers)
        return fail(PKV_EINVAL, "copy_blocks: num_layers %d outside 1..%d", num_layers,
                    pkv::kCopyMaxLayers);
    if (n_pairs < 0) return fail(PKV_EINVAL, "copy_blocks: negative n_pairs");
    if (block_bytes <= 0 || block_bytes % 16 || num_blocks <= 0)
        return fail(PKV_EINVAL, "copy_blocks: block_bytes must be a positive multiple of 16");
    if (!k_caches || !v_caches) return fail(PKV_EINVAL, "copy_blocks: NULL cache arrays");
    for (int32_t l = 0; l < num_layers; ++l) {
        if (!k_caches[l] || !v_caches[l])
            return fail(PKV_EINVAL, "copy_blocks: NULL cache of layer %d", l);
        if ((reinterpret_cast<uintptr_t>(k_caches[l]) | reinterpret_cast<uintptr_t>(v_caches[l])) & 15)
            return fail(PKV_EINVAL, "copy_blocks: caches must be 16-byte aligned");
    }
    if (n_pairs == 0) return pkv::ok();
    if (!pairs) return fail(PKV_EINVAL, "copy_blocks: NULL pairs");
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t l0 = 0; l0 < num_layers; l0 += pkv::kCopyLayers) {
        const int32_t nl = std::min(pkv::kCopyLayers, num_layers - l0);
        pkv::CopyArgs a{};
        for (int32_t l = 0; l < nl; ++l) {
            a.k[l] = static_cast<char*>(k_caches[l0 + l]);
            a.v[l] = static_cast<char*>(v_caches[l0 + l]);
        }
        a.pairs = pairs;
        a.block_bytes = block_bytes;
        a.num_blocks = num_blocks;
        const pkv::LaunchEvents ev = pkv::timer_events(PKV_TIMER_COPY_BLOCKS);
        hipExtLaunchKernelGGL(pkv::copy_blocks_kernel, dim3(unsigned(n_pairs), unsigned(nl), 2),
                              dim3(256), 0, s, ev.start, ev.stop, 0, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return fail(PKV_EHIP, "copy_blocks: launch failed: %s", hipGetErrorString(err));
    }
    return pkv::ok();
}
