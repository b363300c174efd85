// reshape_and_cache: place each new token's K and V rows in the slot the block pool
// gave it. A new token goes into the sequence's current block, a fresh block being
// taken only when the last one is full ("vLLM ve Triton ile maliyet optimizasyonu",
// §03 Yöntem, step 3); this kernel is the device half of that step.
//
// A pure bit copy into K's [blk][g][d/x][BS][x] layout (x = 16 / element_bytes, one
// 16-byte group per row) and V's [blk][g][d][BS] tile. The block size BS = 2^lbs (8, 16
// or 32 tokens) is a run-time argument: slot s is row s % BS of block s / BS. Two forms:
// - flat: one thread per 16-byte group of one (token, KV head). Every wave is busy even
//   for a decode step's few scattered tokens, but a lane's K write lands BS * 16 bytes
//   from its neighbour's and its V elements BS * element_bytes apart;
// - rows (bulk writes: a prompt, a prefill chunk): one wave per 16 consecutive tokens of
//   one KV head, which turns the rows around in LDS so that consecutive lanes write
//   consecutive tokens, i.e. contiguous bytes where the slots are consecutive.
// The launcher takes the rows form when it still gives every compute unit a wave.
// reshape_and_cache_fp8 stores the e4m3 codes of x / scale instead (FP8 KV cache), with
// the same two forms (its rows form: a 256-thread workgroup per tile).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>

#include "device.hpp"
#include "status.hpp"
#include "timer.hpp"

namespace pkv {

template <int E>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const char* __restrict__ key, const char* __restrict__ value, char* __restrict__ kc,
    char* __restrict__ vc, const int32_t* __restrict__ slots, int32_t num_tokens, int32_t hkv,
    int32_t d, int64_t num_blocks, int64_t key_stride_b, int64_t value_stride_b, int32_t lbs) {
    constexpr int X = 16 / E;
    const int bs = 1 << lbs;
    const int nchunk = d / X;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = int64_t(num_tokens) * hkv * nchunk;
    if (idx >= total) return;
    const int c = int(idx % nchunk);
    const int g = int((idx / nchunk) % hkv);
    const int64_t t = idx / (int64_t(nchunk) * hkv);
    // the rows and the slot are independent reads: issue them together
    const int64_t src_k = t * key_stride_b + (int64_t(g) * d + int64_t(c) * X) * E;
    const int64_t src_v = t * value_stride_b + (int64_t(g) * d + int64_t(c) * X) * E;
    const uint4 kv = *reinterpret_cast<const uint4*>(key + src_k);
    const uint4 vv = *reinterpret_cast<const uint4*>(value + src_v);
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= (num_blocks << lbs)) return;
    const int64_t blk = slot >> lbs;
    const int off = int(slot & (bs - 1));
    const int64_t tile = blk * hkv + g;
    *reinterpret_cast<uint4*>(kc + ((tile * nchunk + c) * bs + off) * 16) = kv;
    // V: element k of the group is dimension c*X + k, row `off` of that dimension
    char* vdst = vc + ((tile * d + int64_t(c) * X) * bs + off) * E;
    if constexpr (E == 2) {
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&vv);
#pragma unroll
        for (int k = 0; k < X; ++k) reinterpret_cast<uint16_t*>(vdst + k * bs * E)[0] = h[k];
    } else {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&vv);
#pragma unroll
        for (int k = 0; k < X; ++k) reinterpret_cast<uint32_t*>(vdst + k * bs * E)[0] = w[k];
    }
}

// Rows form: one wave per (16 consecutive tokens, KV head). The rows are read coalesced
// (consecutive lanes take consecutive 16-byte groups of one token), turned around in LDS,
// and written with consecutive lanes on consecutive tokens: for K the same 16-byte group
// of 16 tokens, for V the same dimension of 16 tokens. Tokens with consecutive slots in
// one block (a prompt, a chunk) then write contiguous bytes whatever the block alignment;
// any other slot mapping is still written element by element correctly.
template <int E>
__global__ __launch_bounds__(64) void reshape_and_cache_rows_kernel(
    const char* __restrict__ key, const char* __restrict__ value, char* __restrict__ kc,
    char* __restrict__ vc, const int32_t* __restrict__ slots, int32_t num_tokens, int32_t hkv,
    int32_t d, int64_t num_blocks, int64_t key_stride_b, int64_t value_stride_b, int32_t lbs) {
    constexpr int X = 16 / E;               // elements per 16-byte group
    extern __shared__ uint4 s_rows[];
    const int nchunk = d / X;               // 16-byte groups per row
    const int per = 16 * nchunk;            // groups of the 16 tokens
    const int vpad = nchunk + 1;            // LDS row pitch of V (uint4), padded
    uint4* Kl = s_rows;                     // group c of token r at c * 17 + r
    uint4* Vl = s_rows + nchunk * 17;       // token r's V row at r * vpad
    // KV heads fastest: consecutive workgroups write the head tiles of the same blocks,
    // which lie next to each other in the cache. With heads in the slow dimension, the
    // waves running at once wrote one head's tiles of consecutive blocks, 32 KiB apart
    // (bf16, 8 heads): 3.97 against 6.18 TB/s for 65,536 consecutive slots on MI355X.
    const int64_t wg = blockIdx.x;
    const int g = int(wg % hkv);
    const int64_t t0 = (wg / hkv) * 16;
    const int lane = threadIdx.x;
    const int bs = 1 << lbs;
    // this lane's token for the writes (r = lane % 16) and its slot
    const int rw = lane & 15;
    int64_t slot = t0 + rw < num_tokens ? int64_t(slots[t0 + rw]) : -1;
    if (slot >= (num_blocks << lbs)) slot = -1;
    for (int q = lane; q < per; q += 64) {
        const int r = q / nchunk, c = q - r * nchunk;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (t0 + r < num_tokens) {
            kv = *reinterpret_cast<const uint4*>(key + (t0 + r) * key_stride_b + (int64_t(g) * d + c * X) * E);
            vv = *reinterpret_cast<const uint4*>(value + (t0 + r) * value_stride_b + (int64_t(g) * d + c * X) * E);
        }
        Kl[c * 17 + r] = kv;
        Vl[r * vpad + c] = vv;
    }
    __syncthreads();
    if (slot < 0) return;   // no barrier follows
    const int64_t tile = (slot >> lbs) * hkv + g;
    const int off = int(slot & (bs - 1));
    for (int c = lane >> 4; c < nchunk; c += 4)   // K: group c of token rw
        *reinterpret_cast<uint4*>(kc + ((tile * nchunk + c) * bs + off) * 16) = Kl[c * 17 + rw];
    const char* vrow = reinterpret_cast<const char*>(Vl + rw * vpad);
    for (int i = lane >> 4; i < d; i += 4) {      // V: dimension i of token rw
        char* dst = vc + ((tile * d + i) * bs + off) * E;
        if constexpr (E == 2)
            *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(vrow + i * E);
        else
            *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(vrow + i * E);
    }
}

// FP8 cache: one thread quantises 4 dimensions of one (token, KV head): a quarter of a
// 16-byte K group of the [blk][g][d/16][BS][16] layout (one 4-byte store) and 4 bytes of
// V, one per dimension row of the [blk][g][d][BS] tile. Four dimensions per thread keep
// the correctly rounded divisions per thread few; sixteen made the kernel latency-bound.
template <typename T>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int32_t* __restrict__ slots, int32_t num_tokens, int32_t hkv,
    int32_t d, int64_t num_blocks, int64_t key_stride, int64_t value_stride, float k_scale,
    float v_scale, int32_t lbs) {
    const int bs = 1 << lbs;
    const int nq = d / 4;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = int64_t(num_tokens) * hkv * nq;
    if (idx >= total) return;
    const int c = int(idx % nq);              // dimensions 4c .. 4c + 3
    const int g = int((idx / nq) % hkv);
    const int64_t t = idx / (int64_t(nq) * hkv);
    const uint2 kr = *reinterpret_cast<const uint2*>(key + t * key_stride + int64_t(g) * d + 4 * c);
    const uint2 vr = *reinterpret_cast<const uint2*>(value + t * value_stride + int64_t(g) * d + 4 * c);
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= (num_blocks << lbs)) return;
    const int64_t tile = (slot >> lbs) * hkv + g;
    const int off = int(slot & (bs - 1));
    const uint32_t h[4] = {kr.x & 0xffffu, kr.x >> 16, kr.y & 0xffffu, kr.y >> 16};
    const uint32_t u[4] = {vr.x & 0xffffu, vr.x >> 16, vr.y & 0xffffu, vr.y >> 16};
    uint32_t kw = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) kw |= quantize_fp8(Bits<T>::to_f32(uint16_t(h[k])), k_scale) << (8 * k);
    // dims 4c .. 4c + 3 sit in group 4c / 16 at byte (4c) % 16 of the token's 16-byte row
    *reinterpret_cast<uint32_t*>(kc + ((tile * (d / 16) + (4 * c) / 16) * bs + off) * 16 + (4 * c) % 16) = kw;
    uint8_t* vdst = vc + (tile * d + int64_t(4) * c) * bs + off;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        vdst[k * bs] = uint8_t(quantize_fp8(Bits<T>::to_f32(uint16_t(u[k])), v_scale));
}

// Rows form of the FP8 write (bulk writes), as for the 16-bit caches but with a workgroup
// of 256 threads per 16 consecutive tokens of one KV head: each thread quantises one
// 16-byte chunk (8 dimensions) of K and of V (d = 128), so the correctly rounded divisions
// are spread over four times the threads of a one-wave tile (a wave per tile left the
// launch latency-bound up to a few thousand tokens). Consecutive threads read consecutive
// chunks of a token; the codes are turned around in LDS (K groups at a pitch of 17 x 16
// bytes, V rows at d + 8 bytes: 8-byte aligned, and the 16 rows of one byte column fall in
// 16 different banks) and written one token per thread (thread % 16): 16-byte K groups,
// then single V bytes, so that consecutive slots give contiguous stores.
template <typename T>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_rows_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int32_t* __restrict__ slots, int32_t num_tokens, int32_t hkv,
    int32_t d, int64_t num_blocks, int64_t key_stride, int64_t value_stride, float k_scale,
    float v_scale, int32_t lbs) {
    extern __shared__ uint4 s_codes[];
    const int n8 = d / 8;                    // 16-byte input chunks per row
    const int n16 = d / 16;                  // 16-byte K groups per row
    const int vpitch = d + 8;                // bytes per V row in LDS
    uint8_t* Kl = reinterpret_cast<uint8_t*>(s_codes);              // group c of token r at (c * 17 + r) * 16
    uint8_t* Vl = Kl + n16 * 17 * 16;                                 // token r's codes at r * vpitch
    const int g = blockIdx.y;
    const int64_t t0 = int64_t(blockIdx.x) * 16;
    const int tid = threadIdx.x;
    const int bs = 1 << lbs;
    const int rw = tid & 15;   // the token this thread writes
    int64_t slot = t0 + rw < num_tokens ? int64_t(slots[t0 + rw]) : -1;
    if (slot >= (num_blocks << lbs)) slot = -1;
    const int nt = blockDim.x;
    auto codes8 = [](uint4 a, float scale) {
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
        uint32_t o[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint32_t lo = w[2 * k], hi = w[2 * k + 1];
            o[k] = quantize_fp8(Bits<T>::to_f32(uint16_t(lo)), scale) |
                   (quantize_fp8(Bits<T>::to_f32(uint16_t(lo >> 16)), scale) << 8) |
                   (quantize_fp8(Bits<T>::to_f32(uint16_t(hi)), scale) << 16) |
                   (quantize_fp8(Bits<T>::to_f32(uint16_t(hi >> 16)), scale) << 24);
        }
        return make_uint2(o[0], o[1]);
    };
    for (int q = tid; q < 16 * n8; q += nt) {
        const int r = q / n8, c = q - r * n8;
        uint2 kq = make_uint2(0, 0), vq = make_uint2(0, 0);
        if (t0 + r < num_tokens) {
            const int64_t col = int64_t(g) * d + 8 * c;
            kq = codes8(*reinterpret_cast<const uint4*>(key + (t0 + r) * key_stride + col), k_scale);
            vq = codes8(*reinterpret_cast<const uint4*>(value + (t0 + r) * value_stride + col), v_scale);
        }
        *reinterpret_cast<uint2*>(Kl + ((c >> 1) * 17 + r) * 16 + 8 * (c & 1)) = kq;
        *reinterpret_cast<uint2*>(Vl + r * vpitch + 8 * c) = vq;
    }
    __syncthreads();
    if (slot < 0) return;   // no barrier follows
    const int64_t tile = (slot >> lbs) * hkv + g;
    const int off = int(slot & (bs - 1));
    for (int c = tid >> 4; c < n16; c += nt / 16)   // K: group c of token rw
        *reinterpret_cast<uint4*>(kc + ((tile * n16 + c) * bs + off) * 16) =
            *reinterpret_cast<const uint4*>(Kl + (c * 17 + rw) * 16);
    for (int i = tid >> 4; i < d; i += nt / 16)    // V: dimension i of token rw
        vc[(tile * d + i) * bs + off] = Vl[rw * vpitch + i];
}

}  // namespace pkv

extern "C" int reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                     void* v_cache, const int32_t* slot_mapping,
                                     int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int64_t num_blocks, int64_t key_stride,
                                     int64_t value_stride, int32_t in_dtype, float k_scale,
                                     float v_scale, void* stream) {
    using pkv::fail;
    if (in_dtype != PKV_F16 && in_dtype != PKV_BF16)
        return fail(in_dtype == PKV_F32 ? PKV_ENOTSUP : PKV_EINVAL,
                    "reshape_and_cache_fp8: in_dtype must be F16 or BF16, got %d", in_dtype);
    if (num_tokens < 0) return fail(PKV_EINVAL, "reshape_and_cache_fp8: negative num_tokens");
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PKV_EINVAL, "reshape_and_cache_fp8: block_size must be 8, 16 or 32, got %d",
                    block_size);
    const int lbs = block_size == 8 ? 3 : block_size == 16 ? 4 : 5;
    if (num_kv_heads <= 0 || head_dim <= 0 || head_dim % 16 != 0 || num_blocks <= 0)
        return fail(PKV_EINVAL, "reshape_and_cache_fp8: bad shape (Hkv %d, head_dim %d, "
                                "blocks %lld)", num_kv_heads, head_dim, (long long)num_blocks);
    if (key_stride < int64_t(num_kv_heads) * head_dim ||
        value_stride < int64_t(num_kv_heads) * head_dim || key_stride % 8 || value_stride % 8)
        return fail(PKV_EINVAL, "reshape_and_cache_fp8: token strides must cover Hkv*head_dim "
                                "and be multiples of 8 elements");
    if (!(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
        return fail(PKV_EINVAL, "reshape_and_cache_fp8: k_scale and v_scale must be finite and "
                                "positive");
    if (num_tokens == 0) return pkv::ok();
    if (!key || !value || !k_cache || !v_cache || !slot_mapping)
        return fail(PKV_EINVAL, "reshape_and_cache_fp8: NULL pointer");
    if ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) |
         reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
        return fail(PKV_EINVAL, "reshape_and_cache_fp8: buffers must be 16-byte aligned");
    const int64_t total = int64_t(num_tokens) * num_kv_heads * (head_dim / 4);
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffff) return fail(PKV_EINVAL, "reshape_and_cache_fp8: too many tokens");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* kp = static_cast<const uint16_t*>(key);
    const uint16_t* vp = static_cast<const uint16_t*>(value);
    uint8_t* kcp = static_cast<uint8_t*>(k_cache);
    uint8_t* vcp = static_cast<uint8_t*>(v_cache);
    const pkv::LaunchEvents ev = pkv::timer_events(PKV_TIMER_CACHE_WRITE);
    // rows form when it gives every compute unit a workgroup
    const int64_t rtiles = (int64_t(num_tokens) + 15) / 16;
    const size_t rlds = size_t(head_dim / 16) * 17 * 16 + size_t(16) * (head_dim + 8);
    if (rtiles * num_kv_heads >= pkv::device_cus() && rtiles <= 0x7fffffff &&
        num_kv_heads <= 65535 && rlds <= 65536) {
        const dim3 rgrid{unsigned(rtiles), unsigned(num_kv_heads), 1u};
        if (in_dtype == PKV_BF16)
            hipExtLaunchKernelGGL(pkv::reshape_and_cache_fp8_rows_kernel<pkv::bf16_t>, rgrid,
                                  dim3(256), rlds, s, ev.start, ev.stop, 0, kp, vp, kcp, vcp,
                                  slot_mapping, num_tokens, num_kv_heads, head_dim, num_blocks,
                                  key_stride, value_stride, k_scale, v_scale, lbs);
        else
            hipExtLaunchKernelGGL(pkv::reshape_and_cache_fp8_rows_kernel<pkv::f16_t>, rgrid,
                                  dim3(256), rlds, s, ev.start, ev.stop, 0, kp, vp, kcp, vcp,
                                  slot_mapping, num_tokens, num_kv_heads, head_dim, num_blocks,
                                  key_stride, value_stride, k_scale, v_scale, lbs);
    } else if (in_dtype == PKV_BF16)
        hipExtLaunchKernelGGL(pkv::reshape_and_cache_fp8_kernel<pkv::bf16_t>, dim3(unsigned(grid)),
                              dim3(256), 0, s, ev.start, ev.stop, 0, kp, vp, kcp, vcp,
                              slot_mapping, num_tokens, num_kv_heads, head_dim, num_blocks,
                              key_stride, value_stride, k_scale, v_scale, lbs);
    else
        hipExtLaunchKernelGGL(pkv::reshape_and_cache_fp8_kernel<pkv::f16_t>, dim3(unsigned(grid)),
                              dim3(256), 0, s, ev.start, ev.stop, 0, kp, vp, kcp, vcp,
                              slot_mapping, num_tokens, num_kv_heads, head_dim, num_blocks,
                              key_stride, value_stride, k_scale, v_scale, lbs);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PKV_EHIP, "reshape_and_cache_fp8: launch failed: %s", hipGetErrorString(err));
    return pkv::ok();
}

extern "C" int reshape_and_cache(const void* key, const void* value, void* k_cache,
                                 void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                                 int32_t dtype, void* stream) {
    using pkv::fail;
    const int e = pkv::elem_bytes(dtype);
    if (e == 0) return fail(PKV_EINVAL, "reshape_and_cache: unknown dtype %d", dtype);
    if (num_tokens < 0) return fail(PKV_EINVAL, "reshape_and_cache: negative num_tokens");
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PKV_EINVAL, "reshape_and_cache: block_size must be 8, 16 or 32, got %d",
                    block_size);
    const int lbs = block_size == 8 ? 3 : block_size == 16 ? 4 : 5;
    const int x = 16 / e;
    if (num_kv_heads <= 0 || head_dim <= 0 || head_dim % x != 0 || num_blocks <= 0)
        return fail(PKV_EINVAL, "reshape_and_cache: bad shape (Hkv %d, head_dim %d, blocks %lld)",
                    num_kv_heads, head_dim, (long long)num_blocks);
    if (key_stride < int64_t(num_kv_heads) * head_dim ||
        value_stride < int64_t(num_kv_heads) * head_dim || key_stride % x || value_stride % x)
        return fail(PKV_EINVAL, "reshape_and_cache: token strides must cover Hkv*head_dim and be "
                                "multiples of %d elements", x);
    if (num_tokens == 0) return pkv::ok();
    if (!key || !value || !k_cache || !v_cache || !slot_mapping)
        return fail(PKV_EINVAL, "reshape_and_cache: NULL pointer");
    if ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) |
         reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
        return fail(PKV_EINVAL, "reshape_and_cache: buffers must be 16-byte aligned");
    const int64_t total = int64_t(num_tokens) * num_kv_heads * (head_dim / x);
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffff) return fail(PKV_EINVAL, "reshape_and_cache: too many tokens");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char* kp = static_cast<const char*>(key);
    const char* vp = static_cast<const char*>(value);
    char* kcp = static_cast<char*>(k_cache);
    char* vcp = static_cast<char*>(v_cache);
    const pkv::LaunchEvents ev = pkv::timer_events(PKV_TIMER_CACHE_WRITE);
    // rows form: waves = token tiles x KV heads; LDS = K groups (pitch 17) + V rows
    // (pitch d/x + 1)
    const int64_t rtiles = (int64_t(num_tokens) + 15) / 16;
    const size_t rlds = sizeof(uint4) * size_t(head_dim / x) * (17 + 16) + sizeof(uint4) * 16;
    const bool rows = rtiles * num_kv_heads >= pkv::device_cus() &&
                      rtiles * num_kv_heads <= 0x7fffffff && rlds <= 65536;
    const int64_t kst = key_stride * e, vst = value_stride * e;
    if (rows) {
        const dim3 rgrid{unsigned(rtiles * num_kv_heads), 1u, 1u};
        if (e == 2)
            hipExtLaunchKernelGGL(pkv::reshape_and_cache_rows_kernel<2>, rgrid, dim3(64), rlds, s,
                                  ev.start, ev.stop, 0, kp, vp, kcp, vcp, slot_mapping, num_tokens,
                                  num_kv_heads, head_dim, num_blocks, kst, vst, lbs);
        else
            hipExtLaunchKernelGGL(pkv::reshape_and_cache_rows_kernel<4>, rgrid, dim3(64), rlds, s,
                                  ev.start, ev.stop, 0, kp, vp, kcp, vcp, slot_mapping, num_tokens,
                                  num_kv_heads, head_dim, num_blocks, kst, vst, lbs);
    } else if (e == 2) {
        hipExtLaunchKernelGGL(pkv::reshape_and_cache_kernel<2>, dim3(unsigned(grid)), dim3(256), 0,
                              s, ev.start, ev.stop, 0, kp, vp, kcp, vcp, slot_mapping, num_tokens,
                              num_kv_heads, head_dim, num_blocks, kst, vst, lbs);
    } else {
        hipExtLaunchKernelGGL(pkv::reshape_and_cache_kernel<4>, dim3(unsigned(grid)), dim3(256), 0,
                              s, ev.start, ev.stop, 0, kp, vp, kcp, vcp, slot_mapping, num_tokens,
                              num_kv_heads, head_dim, num_blocks, kst, vst, lbs);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PKV_EHIP, "reshape_and_cache: launch failed: %s", hipGetErrorString(err));
    return pkv::ok();
}
