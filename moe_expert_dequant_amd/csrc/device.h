// device.h -- small gfx950 device helpers shared by the libffnq kernels:
// vector types, the bf16 MFMA, dequant unpackers and exact bf16 rounding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffnq {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// D = A(16x32) * B(32x16) + C with bf16 operands and fp32 accumulation.
// Lane l holds A[l%16][8(l/16)+e] and B[8(l/16)+e][l%16] (e = 0..7, element e
// in half e%2 of register e/2) and receives D[4(l/16)+i][l%16] in register i.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                    c, 0, 0, 0);
}

__device__ __forceinline__ float bf16lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Eight INT4 codes (one dword, input j in nibble j) -> eight bf16 values
// 128 + code.  0x4300 is bf16 128.0 with a mantissa step of 1, so OR-ing a
// code into its low bits is exact.  Register v holds codes (v, v+4), so the
// element order is the permutation [0,4,1,5,2,6,3,7] of the eight inputs.
// Each register is one v_bitop3_b32 ((a & b) | c, truth table 0xEA) after a
// shift.
__device__ __forceinline__ u32x4 unpack_int4_biased(uint32_t w)
{
    u32x4 r;
    r[0] = __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x43004300u, (unsigned char)0xEA);
    r[1] = __builtin_amdgcn_bitop3_b32(w >> 4, 0x000F000Fu, 0x43004300u, (unsigned char)0xEA);
    r[2] = __builtin_amdgcn_bitop3_b32(w >> 8, 0x000F000Fu, 0x43004300u, (unsigned char)0xEA);
    r[3] = __builtin_amdgcn_bitop3_b32(w >> 12, 0x000F000Fu, 0x43004300u, (unsigned char)0xEA);
    return r;
}

// Four int8 codes (one dword) -> two registers of bf16 pairs holding
// q + 128 in natural order.  q + 128 is an integer in [0, 255], which bf16
// (8 significant bits) holds exactly, so its bf16 is the upper half of the
// fp32 conversion.
__device__ __forceinline__ u32x2 unpack_int8_biased(uint32_t w)
{
    uint32_t u = w ^ 0x80808080u;
    float f0 = (float)(u & 0xFFu), f1 = (float)((u >> 8) & 0xFFu);
    float f2 = (float)((u >> 16) & 0xFFu), f3 = (float)(u >> 24);
    u32x2 r;
    r[0] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    r[1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    return r;
}

// Natural-order bf16 (x0..x7 in four registers) -> the [0,4,1,5,2,6,3,7]
// order that unpack_int4_biased produces.
__device__ __forceinline__ u32x4 permute_0415(u32x4 n)
{
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(n[2], n[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(n[2], n[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(n[3], n[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(n[3], n[1], 0x07060302u);
    return r;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// double -> bf16 bits with a single rounding to nearest even, including the
// bf16 subnormal range and overflow to infinity.
__device__ __forceinline__ uint16_t bf16_from_f64(double v)
{
    uint64_t b = (uint64_t)__double_as_longlong(v);
    uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return (uint16_t)(sign | 0x7FC0u);
    int e = (int)(a >> 52) - 1023;
    if (e >= -126) {
        uint64_t lsb = (a >> 45) & 1u;
        a += 0x00000FFFFFFFFFFFull + lsb;           // round half to even at the 8th significant bit
        int e2 = (int)(a >> 52) - 1023;
        if (e2 > 127) return (uint16_t)(sign | 0x7F80u);
        return (uint16_t)(sign | (uint16_t)((e2 + 127) << 7) | (uint16_t)((a >> 45) & 0x7Fu));
    }
    // subnormal bf16: multiples of 2^-133; scaling by 2^133 is exact
    double q = __builtin_rint(__longlong_as_double((long long)a) * 0x1p133);
    return (uint16_t)(sign | (uint16_t)q);
}

// Split an fp32 value into bf16 hi + lo with a == hi + lo to about 2^-17
// relative (exact when a has at most 16 significant bits).
__device__ __forceinline__ void split_bf16(float a, uint16_t& hi, uint16_t& lo)
{
    hi = bf16_rne(a);
    lo = bf16_rne(a - bf16_f32(hi));
}

// The gated activation in fp32 (device exp/tanh).  For g >= 24 both forms
// return g exactly (exp(-g) and 1 - tanh are below half an ulp of 1).
__device__ __forceinline__ float act_f32(int act, float g)
{
    if (act == 1) return g / (1.0f + __expf(-g));
    const float c = 0.7978845608028654f;   // sqrt(2/pi)
    return 0.5f * g * (1.0f + tanhf(c * (g + 0.044715f * g * g * g)));
}

__device__ __forceinline__ double act_f64(int act, double g)
{
    if (act == 1) return g / (1.0 + exp(-g));
    const double c = 0.7978845608028654;   // sqrt(2/pi)
    return 0.5 * g * (1.0 + tanh(c * (g + 0.044715 * g * g * g)));
}


// Direct global->LDS loads (gfx950 global_load_lds_dword / _dwordx4): lane i
// writes its 4 or 16 bytes to LDS byte address lds + i*size.  Issued from
// inline asm so that the compiler's counter bookkeeping covers only the
// loads it sees; the caller waits for these with an explicit
// s_waitcnt vmcnt(N) (loads retire in order) before a barrier.  M0 carries
// the LDS base and is restored afterwards; the base must be wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
        : "memory");
}

__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
        : "memory");
}

}  // namespace ffnq
