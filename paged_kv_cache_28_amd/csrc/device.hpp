// Device-side helpers for the gfx950 kernels: element types, conversions with
// round-to-nearest-even, the exp2 instruction, and the matrix-instruction wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Storage tags: the caches hold raw 16-bit patterns.
struct bf16_t {};
struct f16_t {};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// The index of the calling wave in its workgroup, as a value the compiler knows to be the
// same in every lane (loops bounded by it compile to scalar loops).
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
}

// Loads of K/V tile data that a decode launch reads exactly once: non-temporal
// (global_load ... nt), so the L2 and the Infinity Cache do not keep lines that will not be
// read again. On MI355X this streamed the 8B batch's tile set 6-10% faster than plain loads
// (the gather ceilings that bench.py measures), and a contiguous read likewise.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_once16(const void* p) {
    const u32x4_t r = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
    return make_uint4(r[0], r[1], r[2], r[3]);
}
__device__ __forceinline__ uint2 ld_once8(const void* p) {
    const u32x2_t r = __builtin_nontemporal_load(static_cast<const u32x2_t*>(p));
    return make_uint2(r[0], r[1]);
}
__device__ __forceinline__ uint32_t ld_once4(const void* p) {
    return __builtin_nontemporal_load(static_cast<const unsigned int*>(p));
}

// Block ids are valid in [0, num_blocks). As a 32-bit unsigned limit (negative ids wrap past
// it) the per-tile test is one scalar compare; a 64-bit signed compare has no scalar form
// here and went through vector registers that loads in flight were still filling, which
// made the compiler wait for them before the next tile's loads.
__device__ __forceinline__ uint32_t block_limit(int64_t num_blocks) {
    return num_blocks <= 0 ? 0u : (num_blocks > int64_t(0x7fffffff) ? 0x80000000u : uint32_t(num_blocks));
}

// The same non-temporal tile loads through a buffer resource: a scalar descriptor over one
// (block, KV head) tile of `bytes` bytes, against which each lane takes a fixed byte offset.
// Moving to the next tile then rewrites scalar registers only. With 64-bit per-lane
// addresses the compiler recomputed the address registers at the head of the tile loop and,
// sharing them with registers that loads were still filling, waited for every outstanding
// load there: the next tile was requested only once the current one had arrived, which
// left one tile in flight while the matrix products ran. Offsets past `bytes` would read
// zero; none is formed. Descriptor word 3 is the raw-dword format of this GPU family.
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
constexpr int kBufNT = 2;   // cache policy of the load: non-temporal
__device__ __forceinline__ buf_rsrc_t tile_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), bytes, 0x00020000);
}
// POL: the cache policy (kBufNT; 0 for plain loads, where another wave reads the rest of
// the same lines, as the two halves of a 32-token block are).
template <int POL = kBufNT>
__device__ __forceinline__ uint4 bld16(buf_rsrc_t r, int off, int soff = 0) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, POL);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int POL = kBufNT>
__device__ __forceinline__ uint2 bld8(buf_rsrc_t r, int off, int soff = 0) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, POL);
    return make_uint2(v[0], v[1]);
}
template <int POL = kBufNT>
__device__ __forceinline__ uint32_t bld4(buf_rsrc_t r, int off, int soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, POL);
}

// fp32 -> 16-bit patterns, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    // The empty asm pins f as an fp32 value: without it the compiler may fuse the
    // multiply that produced f into the conversion (v_fma_mix*), rounding once from
    // the exact product instead of from the fp32 result.
    asm("" : "+v"(f));
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, uint32_t(h) << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Output stores in the three supported output types.
template <typename OutT> struct OutStore;
// st4 writes elements i .. i + 3 (i a multiple of 4, base 16-byte aligned) in one store.
template <> struct OutStore<float> {
    __device__ __forceinline__ static void st(void* base, int64_t i, float v) {
        static_cast<float*>(base)[i] = v;
    }
    __device__ __forceinline__ static void st4(void* base, int64_t i, float4 v) {
        *reinterpret_cast<float4*>(static_cast<float*>(base) + i) = v;
    }
};
template <> struct OutStore<bf16_t> {
    __device__ __forceinline__ static void st(void* base, int64_t i, float v) {
        static_cast<uint16_t*>(base)[i] = f32_to_bf16_bits(v);
    }
    __device__ __forceinline__ static void st4(void* base, int64_t i, float4 v) {
        const uint2 w = make_uint2(uint32_t(f32_to_bf16_bits(v.x)) | (uint32_t(f32_to_bf16_bits(v.y)) << 16),
                                   uint32_t(f32_to_bf16_bits(v.z)) | (uint32_t(f32_to_bf16_bits(v.w)) << 16));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + i) = w;
    }
};
template <> struct OutStore<f16_t> {
    __device__ __forceinline__ static void st(void* base, int64_t i, float v) {
        static_cast<uint16_t*>(base)[i] = f32_to_f16_bits(v);
    }
    __device__ __forceinline__ static void st4(void* base, int64_t i, float4 v) {
        const uint2 w = make_uint2(uint32_t(f32_to_f16_bits(v.x)) | (uint32_t(f32_to_f16_bits(v.y)) << 16),
                                   uint32_t(f32_to_f16_bits(v.z)) | (uint32_t(f32_to_f16_bits(v.w)) << 16));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + i) = w;
    }
};

// Matrix-instruction wrappers per input type.
//   qk(a, b, c):  16x16x32, A and B are 8 elements per lane (one uint4)
//   pv(a, b, c):  16x16x16, A and B are 4 elements per lane (one uint2)
//   split(p, hi, lo): p ~= hi + lo with both parts in the input type, so the
//                     probabilities keep ~16 significant bits through the product
template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
    __device__ __forceinline__ static f32x4 qk(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 pv(uint2 a, uint2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                         __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
    }
    // p is finite here, so the hardware conversion (round to nearest even) applies.
    __device__ __forceinline__ static void split(float p, uint16_t& hi, uint16_t& lo) {
        hi = __builtin_bit_cast(uint16_t, (__bf16)p);
        lo = __builtin_bit_cast(uint16_t, (__bf16)(p - bf16_bits_to_f32(hi)));
    }
};

template <> struct Mfma<f16_t> {
    __device__ __forceinline__ static f32x4 qk(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 pv(uint2 a, uint2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static void split(float p, uint16_t& hi, uint16_t& lo) {
        hi = f32_to_f16_bits(p);
        lo = f32_to_f16_bits(p - f16_bits_to_f32(hi));
    }
};

// 16-bit pattern of the input type -> fp32 (exact).
template <typename T> struct Bits;
template <> struct Bits<bf16_t> {
    __device__ __forceinline__ static float to_f32(uint16_t h) { return bf16_bits_to_f32(h); }
};
template <> struct Bits<f16_t> {
    __device__ __forceinline__ static float to_f32(uint16_t h) { return f16_bits_to_f32(h); }
};

// ---- FP8 KV cache: OCP e4m3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// S.1111.111 = NaN, largest finite 448).
//
// fp8x4_to<T>(w): the four codes in w (lowest byte first) as four 16-bit values of T,
// two per 32-bit word, lowest first. Exact: every e4m3 value is a bf16 and an fp16
// value. One gfx950 conversion per pair; its scale operand is 1 (the cache scales are
// applied to the logits and the output instead).
template <typename T> struct Fp8;
template <> struct Fp8<bf16_t> {
    __device__ __forceinline__ static uint2 x4(uint32_t w) {
        return make_uint2(
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
    }
};
template <> struct Fp8<f16_t> {
    __device__ __forceinline__ static uint2 x4(uint32_t w) {
        return make_uint2(
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)));
    }
};

// binary32 -> e4m3 code: the nearest finite value, ties to the even code. Magnitudes
// beyond 448 (infinities too) saturate: the hardware conversion (round to nearest even)
// only ever sees the clamped value. NaN gives S.1111.111 with the input's sign.
__device__ __forceinline__ uint32_t f32_to_fp8(float x) {
    const float c = fminf(fmaxf(x, -448.0f), 448.0f);
    const uint32_t code = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false)) & 0xffu;
    return x != x ? ((__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u) | 0x7fu : code;
}

// The stored code of input element x under a per-tensor scale: x / scale rounded once
// to binary32 (an IEEE division), then encoded.
__device__ __forceinline__ uint32_t quantize_fp8(float x, float scale) {
    return f32_to_fp8(x / scale);
}

// Codes of the 16 input elements in a0 (elements 0-7) and a1 (8-15), packed four per
// word, lowest first: one 16-byte group of the FP8 cache.
template <typename T>
__device__ __forceinline__ uint4 quantize_fp8_x16(uint4 a0, uint4 a1, float scale) {
    const uint32_t w[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[2 * k], hi = w[2 * k + 1];
        o[k] = quantize_fp8(Bits<T>::to_f32(uint16_t(lo)), scale) |
               (quantize_fp8(Bits<T>::to_f32(uint16_t(lo >> 16)), scale) << 8) |
               (quantize_fp8(Bits<T>::to_f32(uint16_t(hi)), scale) << 16) |
               (quantize_fp8(Bits<T>::to_f32(uint16_t(hi >> 16)), scale) << 24);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, 64));
}

// max over the four lanes l, l^16, l^32, l^48 with the gfx950 row-swap instructions:
// permlane16_swap exchanges the odd 16-lane rows of one operand with the even rows of
// the other, permlane32_swap the upper half of one with the lower half of the other;
// fed the same value twice, each yields the pair {x[l], x[l^16]} (resp. x[l^32]).
__device__ __forceinline__ float max_over_rows(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__builtin_bit_cast(float, (unsigned)r16[0]),
                          __builtin_bit_cast(float, (unsigned)r16[1]));
    const unsigned v = __builtin_bit_cast(unsigned, y);
    auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r32[0]),
                 __builtin_bit_cast(float, (unsigned)r32[1]));
}

// Host side: compute units of the current device (cached per device; 256 when the
// query fails). Launchers size grids and plans by it.
int device_cus();

}  // namespace pkv
