// Device-side helpers shared by the gfx950 kernels of the LSH-attention forward.
//
// MFMA conventions (CDNA3/CDNA4 32x32 tiles, wave64):
//   D[32x32] += A[32xK] * B[Kx32], K = 2*KPL per instruction.
//   lane l:  A operand = row  (l % 32), k = KPL*(l / 32) + [0, KPL)
//            B operand = col  (l % 32), k = KPL*(l / 32) + [0, KPL)
//            D element j (0..15) = row 8*(j/4) + 4*(l/32) + (j%4), col (l % 32)
// bf16 uses v_mfma_f32_32x32x16_bf16 (KPL = 8), f32 uses v_mfma_f32_32x32x2_f32
// (KPL = 1).  The contraction only needs A and B to agree on which k each
// (lane, slot) holds, so any consistent permutation of k is allowed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lshk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Storage type of bfloat16 tensors in memory.
struct bf16_t { uint16_t bits; };

template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
    static constexpr int KPL = 8;          // elements per lane per instruction
    static constexpr int KSTEP = 16;       // k per instruction
    typedef bf16x8 Frag;
    static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // 8 consecutive elements from 16-byte-aligned memory (global or LDS).
    static __device__ __forceinline__ Frag load(const bf16_t* p) {
        return *reinterpret_cast<const Frag*>(p);
    }
    static __device__ __forceinline__ Frag zero() { return Frag{}; }
};

template <> struct Mfma<float> {
    static constexpr int KPL = 1;
    static constexpr int KSTEP = 2;
    typedef float Frag;
    static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ Frag load(const float* p) { return *p; }
    static __device__ __forceinline__ Frag zero() { return 0.f; }
};

// 16x16 tiles (wave64): D[16x16] += A[16xK] * B[Kx16], K = 4*KPL per instruction.
//   lane l: A operand = row (l % 16), k = KPL*(l / 16) + [0, KPL)
//           B operand = col (l % 16), k = KPL*(l / 16) + [0, KPL)
//           D element j (0..3) = row 4*(l/16) + j, col (l % 16)
// bf16: v_mfma_f32_16x16x32_bf16 (KPL = 8); f32: v_mfma_f32_16x16x4_f32 (KPL = 1).
template <typename T> struct Mfma16;

template <> struct Mfma16<bf16_t> {
    static constexpr int KPL = 8;
    static constexpr int KSTEP = 32;
    typedef bf16x8 Frag;
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ Frag load(const bf16_t* p) {
        return *reinterpret_cast<const Frag*>(p);
    }
};

template <> struct Mfma16<float> {
    static constexpr int KPL = 1;
    static constexpr int KSTEP = 4;
    typedef float Frag;
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ Frag load(const float* p) { return *p; }
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two floats -> two bfloat16 packed in a word (v_cvt_pk_bf16_f32: round to
// nearest even; low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// Rows held in the 16x16 MFMA output layout: lane (r16 = lane & 15, g = lane >> 4)
// holds, for each 16-wide d tile dt, the 4 values d = 16 dt + 4 g .. + 3 of row
// r16.  For a pair of tiles (dt0, dt0 + 1) given as packed bf16 words (a0, a1)
// and (b0, b1), lanes g and g ^ 1 (lane ^ 16, the same row) trade one half, so
// that each lane stores 16 contiguous bytes: the even lane d 16 dt0 + 4 g .. +7,
// the odd lane d 16 (dt0 + 1) + 4 (g - 1) .. +7.  A store instruction then
// writes 64 bytes of each of 16 rows instead of 32, and there are half as
// many.  Every lane of the wave must call it (the trade reads lane ^ 16).
__device__ __forceinline__ void store_tile_pair_bf16(bf16_t* row, int g, int dt0, uint32_t a0,
                                                     uint32_t a1, uint32_t b0, uint32_t b1)
{
    const bool odd = (g & 1) != 0;
    const uint32_t r0 = (uint32_t)__shfl_xor((int)(odd ? a0 : b0), 16);
    const uint32_t r1 = (uint32_t)__shfl_xor((int)(odd ? a1 : b1), 16);
    const u32x4 w = odd ? u32x4{r0, r1, b0, b1} : u32x4{a0, a1, r0, r1};
    const int d0 = odd ? 16 * (dt0 + 1) + 4 * (g - 1) : 16 * dt0 + 4 * g;
    *reinterpret_cast<u32x4*>(row + d0) = w;
}

__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return bf16_t{f32_to_bf16_rne(f)}; }
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Device-side bounds checks.  The kernels clamp or skip every index they take
// from caller data (positions read from perm, bucket ids, sorted slots), so a
// bad value never leaves a buffer.  A build with LSH_DEVICE_CHECKS defined also
// counts each such value: LSH_CHECK(cond) adds one to this translation unit's
// device counter when cond is false (a bad value may be counted by more than
// one check), and LSH_CHECK_ACCESSOR(fn) defines the host function that adds
// the counter to *acc and optionally clears it.  Without the macro both are
// empty and the kernels are unchanged.
#ifdef LSH_DEVICE_CHECKS
static __device__ unsigned int g_check_failures;
#define LSH_CHECK(cond)                                                                     \
    do {                                                                                    \
        if (!(cond)) atomicAdd(&::lshk::g_check_failures, 1u);                              \
    } while (0)
#define LSH_CHECK_ACCESSOR(fn)                                                              \
    hipError_t fn(unsigned long long* acc, bool reset)                                      \
    {                                                                                       \
        unsigned int v = 0;                                                                 \
        hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_failures), sizeof v);     \
        if (e != hipSuccess) return e;                                                      \
        *acc += v;                                                                          \
        if (!reset) return hipSuccess;                                                      \
        const unsigned int zero = 0;                                                        \
        return hipMemcpyToSymbol(HIP_SYMBOL(g_check_failures), &zero, sizeof zero);         \
    }
#else
#define LSH_CHECK(cond) ((void)0)
#define LSH_CHECK_ACCESSOR(fn)                                                              \
    hipError_t fn(unsigned long long*, bool) { return hipSuccess; }
#endif

}  // namespace lshk
