// Device helpers shared by the gfx950 kernels: vector types, exact storage
// conversions, wave-level shuffles.
#pragma once

#include "../internal.h"

namespace da {
namespace dev {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;     // nearest, ties to even
}
__device__ __forceinline__ float f16_to_f32(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ uint32_t f32_to_f16(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);  // nearest, ties to even
}

template <int F>
__device__ __forceinline__ float load_scalar(const void *p, int64_t i) {
    if constexpr (F == FMT_F32) return ((const float *)p)[i];
    else if constexpr (F == FMT_F16) return f16_to_f32(((const uint16_t *)p)[i]);
    else return bf16_to_f32(((const uint16_t *)p)[i]);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One data-parallel-primitive move: lane i takes `v` of the lane that the
// row-local pattern CTRL names (VALU, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// One butterfly step of a lane reduction on the VALU: op(x, x of lane
// i ^ MASK) in every lane i, for a commutative op on a 32-bit value.
// Masks 1, 2 and 8 are single row moves (quad_perm [1,0,3,2], [2,3,0,1],
// row_ror:8); mask 4 is a mirror within 8 lanes followed by a reversal
// within 4 (lane i ends with lane i ^ 4); masks 16 and 32 use
// v_permlane16_swap / v_permlane32_swap of x with itself, whose two
// outputs then hold, in every lane, x of the lane and of its partner, in
// some order.  Each lane gets exactly op(x, __shfl_xor(x, MASK)), without
// the LDS round trip of ds_bpermute.
// x of lane i ^ MASK, for MASK 1, 2, 4 or 8 (row moves, as in xor_step).
template <int MASK>
__device__ __forceinline__ float lane_xor(float x) {
    static_assert(MASK == 1 || MASK == 2 || MASK == 4 || MASK == 8, "row-local lane mask");
    int v = __float_as_int(x);
    if constexpr (MASK == 1) v = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    if constexpr (MASK == 2) v = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    if constexpr (MASK == 4) {
        v = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);   // row_half_mirror
        v = __builtin_amdgcn_mov_dpp(v, 0x1B, 0xF, 0xF, false);    // quad_perm [3,2,1,0]
    }
    if constexpr (MASK == 8) v = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);  // row_ror:8
    return __int_as_float(v);
}

template <int MASK, typename T, typename Op>
__device__ __forceinline__ T xor_step(T x, Op op) {
    static_assert(sizeof(T) == 4, "32-bit lanes");
    static_assert(MASK == 1 || MASK == 2 || MASK == 4 || MASK == 8 || MASK == 16 || MASK == 32, "lane mask");
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    if constexpr (MASK >= 16) {
        const auto pr = MASK == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                                   : __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return op(__builtin_bit_cast(T, (uint32_t)pr[0]), __builtin_bit_cast(T, (uint32_t)pr[1]));
    } else {
        return op(x, __builtin_bit_cast(T, __float_as_uint(lane_xor<MASK>(__uint_as_float(u)))));
    }
}
// Butterfly steps for masks FIRST, 2 FIRST, ... below END (powers of two).
template <int FIRST, int END, typename T, typename Op>
__device__ __forceinline__ T xor_reduce(T x, Op op) {
    if constexpr (FIRST < END) {
        x = xor_step<FIRST>(x, op);
        return xor_reduce<2 * FIRST, END>(x, op);
    } else {
        return x;
    }
}
struct OpAdd {
    __device__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpMin {
    __device__ float operator()(float a, float b) const { return fminf(a, b); }
};
struct OpOr {
    __device__ int operator()(int a, int b) const { return a | b; }
};

// Maximum over the 16 lanes of each row, left in every lane of the row: swap
// neighbours, swap pairs, mirror within 8 lanes, mirror within 16 lanes.
// Maximum is exact, so the result equals that of any reduction order.
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));    // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_mov<0x4E>(x));    // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_mov<0x141>(x));   // row_half_mirror
    x = fmaxf(x, dpp_mov<0x140>(x));   // row_mirror
    return x;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// Buffer resource over [base, base + bytes): loads through it use 32-bit
// lane offsets, and any access at or beyond `bytes` returns zeros instead of
// touching memory (hardware range check on the lane offset).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// 16-byte non-temporal (streaming) load through a buffer resource.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 2);
}

// Hide a value's known bits from the optimiser (no instruction is emitted).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
// Byte n of x as float (selects v_cvt_f32_ubyte{0..3}).
__device__ __forceinline__ float ubyte_f32(uint32_t x, int n) { return (float)(unsigned char)(x >> (8 * n)); }

// Physical channel fed by MFMA `mf`, lane group g (lane / 16), element e, when
// a lane loads 16 bytes at byte offset 64 * chunk + 16 * g of a row:
//   fp32:  16x16x4 MFMA per element  -> channel 16 * chunk + 4 * g + e (mf = 4 * chunk + e)
//   16-bit: 16x16x32 MFMA per chunk  -> channel 32 * chunk + 8 * g + e (mf = chunk)
//   uint4: 16x16x32 MFMA per dword u of the lane's 16 bytes; the codes of a dword
//          come out as channels {0,4,1,5,2,6,3,7} -> 32 * g + 8 * u + pos(e)
template <int KF>
__device__ __forceinline__ int qk_dim(int mf, int g, int e) {
    if constexpr (KF == FMT_F32) {
        return 16 * (mf >> 2) + 4 * g + (mf & 3);
    } else if constexpr (KF == FMT_U4) {
        const int pos = (e >> 1) + 4 * (e & 1);
        return 32 * g + 8 * mf + pos;
    } else {
        return 32 * mf + 8 * g + e;
    }
}

// x split into its `s`-th term of the 16-bit MFMA type MT (0 = nearest value,
// then nearest value of the remainder, ...).  The terms sum to x within the
// last term's rounding.
template <int MT>
__device__ __forceinline__ uint32_t split_term(float x, int s) {
    uint32_t bits = 0;
    for (int i = 0; i <= s; ++i) {
        if constexpr (MT == FMT_BF16) { bits = f32_to_bf16(x); x -= bf16_to_f32(bits); }
        else { bits = f32_to_f16(x); x -= f16_to_f32(bits); }
    }
    return bits;
}

}  // namespace dev
}  // namespace da
