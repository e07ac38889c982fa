// gfx950.hpp -- device helpers shared by the gfx950 kernels of libftm: vector
// types, half-precision conversions, raw buffer descriptors, the matrix-core
// operations with their hi/lo operand splits, and small compile-time tools.
// Device code only; each kernel file includes it inside namespace ftm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "ftm_internal.hpp"

namespace ftm {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor word 3 for raw (untyped) buffer access on the gfx9 family.
constexpr int kRsrcWord3 = 0x00020000;

// ---------------------------------------------------------------------------
// Number formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
    return __uint_as_float(h << 16);
}
// fp32 -> binary16, round to nearest even (the hardware's default mode).
__device__ __forceinline__ uint32_t float_to_half_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
// fp32 -> bfloat16, round to nearest even on the integer pattern; NaN maps
// to the canonical quiet NaN with its sign.
__device__ __forceinline__ uint32_t float_to_bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Buffer descriptor over [base, base + bytes).  Both are the same across the
// wave; readfirstlane states that, so the descriptor sits in scalar
// registers instead of being rebuilt per lane around every load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), (short)0, n, kRsrcWord3);
}

// 16 bytes per lane from a buffer straight into LDS: lane i of the wave
// writes bytes lds + 16 i .. +15 (lds is the same for the whole wave).
// Offsets past the buffer's end read zero.
// The byte offset is voffset (per lane) + soffset (the same for the wave).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds, int voffset, int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset, 0, 0);
}

// 4 bytes per lane from a buffer straight into LDS: lane i of the wave
// writes bytes lds + 4 i .. +3.
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t rsrc, void* lds, int voffset, int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 4, voffset, soffset, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight fp16 or bf16 values in a 16-byte vector, as fp32.
template <int KV> struct Elem16 {
    __device__ static void unpack(const u32x4 w, float* x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (KV == KV_BF16) {
                x[2 * i] = __uint_as_float(w[i] << 16);
                x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            } else {
                x[2 * i] = half_bits_to_float(w[i] & 0xffffu);
                x[2 * i + 1] = half_bits_to_float(w[i] >> 16);
            }
        }
    }
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int KV> struct Mfma;
template <> struct Mfma<KV_BF16> {
    typedef bf16x8 vec8;
    typedef s16x4 vec4;
    __device__ static vec8 bits8(const u32x4 w) { return __builtin_bit_cast(vec8, w); }
    __device__ static vec4 bits4(const u32x2 w) { return __builtin_bit_cast(vec4, w); }
    __device__ static void split8(const float* x, vec8& hi, vec8& lo) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const __bf16 h = (__bf16)x[i];
            hi[i] = h;
            lo[i] = (__bf16)(x[i] - (float)h);
        }
    }
    __device__ static void split4(const float* x, vec4& hi, vec4& lo) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const __bf16 h = (__bf16)x[i];
            hi[i] = __builtin_bit_cast(short, h);
            lo[i] = __builtin_bit_cast(short, (__bf16)(x[i] - (float)h));
        }
    }
    __device__ static f32x4 mma32(const vec8 a, const vec8 b, const f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x4 mma16(const vec4 a, const vec4 b, const f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<KV_F16> {
    typedef f16x8 vec8;
    typedef f16x4 vec4;
    __device__ static vec8 bits8(const u32x4 w) { return __builtin_bit_cast(vec8, w); }
    __device__ static vec4 bits4(const u32x2 w) { return __builtin_bit_cast(vec4, w); }
    __device__ static void split8(const float* x, vec8& hi, vec8& lo) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 h = (_Float16)x[i];
            hi[i] = h;
            lo[i] = (_Float16)(x[i] - (float)h);
        }
    }
    __device__ static void split4(const float* x, vec4& hi, vec4& lo) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const _Float16 h = (_Float16)x[i];
            hi[i] = h;
            lo[i] = (_Float16)(x[i] - (float)h);
        }
    }
    __device__ static f32x4 mma32(const vec8 a, const vec8 b, const f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x4 mma16(const vec4 a, const vec4 b, const f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
};

// Reduction over the four lanes l % 16 + 16 r (r = 0..3) that share a
// column of a 16x16 matrix-core result.  v_permlane16_swap exchanges rows
// 0<->1 and 2<->3 of two copies of x, v_permlane32_swap the two halves of
// the wave; each step leaves the lane with its own value and its partner's,
// so every lane of a column ends with the same result.
template <typename Op>
__device__ __forceinline__ float column_reduce(float x, Op op) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(x);
    const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float column_max(float x) {
    return column_reduce(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float column_sum(float x) {
    return column_reduce(x, [](float a, float b) { return a + b; });
}

// ---------------------------------------------------------------------------
// Cross-lane reductions.  A row of data is held by LPR consecutive lanes
// (LPR in {4, 8, 16, 32}); the all-reduce over those lanes stays inside a
// DPP row where it can: quad swaps, then the half-row mirror (8 lanes) or
// rotations by 4 and 8 (16 lanes); a 32-lane row adds one cross-row swap.
// ---------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

template <int LPR> __device__ __forceinline__ float group_sum(float v) {
    v += dpp<kQuadSwap1>(v);
    v += dpp<kQuadSwap2>(v);
    if constexpr (LPR == 8) v += dpp<kRowHalfMirror>(v);
    if constexpr (LPR >= 16) {
        v += dpp<kRowRor4>(v);
        v += dpp<kRowRor8>(v);
    }
    if constexpr (LPR == 32) v += __shfl_xor(v, 16);
    return v;
}
// Orders this wave's LDS accesses: everything issued before has completed.
__device__ __forceinline__ void lds_wave_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

}  // namespace
}  // namespace ftm
