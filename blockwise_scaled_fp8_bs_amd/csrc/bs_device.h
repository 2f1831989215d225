// Device-side arithmetic shared by the quantizer kernels and their
// diagnostics: bf16 unpacking, the block scale, the element quotient and the
// e4m3 encode.  gfx950 only.
//
// The quantization of one block (pages: "[not for land] float8 blockwise
// scaling training prototype using deep_gemm", description; "add FSDP and TP
// tests for Float8BlockwiseLinear", review thread on the kernel module for
// EPS = 1e-12):
//     s = fl32(max(amax, EPS) / 448),   y = fl32(x / s),
//     q = e4m3_rne(clamp(y, -448, 448)).
// Both divisions must be the correctly rounded IEEE quotient.  They are
// evaluated here with short fma sequences instead of the ~10-instruction
// IEEE divide; bs_diag_division proves on the device that the sequences give
// the IEEE quotient bit for bit over every (amax, x) pair that bf16 inputs
// can produce, and the parity tests compare against the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bs {

constexpr float kEps = 1e-12f;          // floor on the block amax
constexpr float kE4m3Max = 448.0f;      // largest finite e4m3 magnitude
constexpr float kInv448 = 1.0f / 448.0f;  // RN(1/448), folded by the compiler

// bf16 halves of a 32-bit word (little endian: element 0 in the low half).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Block scale s = fl32(max(amax, EPS) / 448) and r ~ 1/s.
// s: one Markstein step on the constant divisor 448 (quotient estimate
// a * RN(1/448), exact remainder by fma, corrected quotient by fma).
// r: hardware reciprocal refined by one Newton step.
struct Scale {
    float s;
    float r;
};

__device__ __forceinline__ Scale block_scale(float amax) {
    const float a = fmaxf(amax, kEps);
    float s = a * kInv448;
    const float rem = __builtin_fmaf(-s, kE4m3Max, a);
    s = __builtin_fmaf(rem, kInv448, s);
    float r = __builtin_amdgcn_rcpf(s);
    r = __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
    return {s, r};
}

// y = fl32(x / s) given r ~ 1/s: quotient estimate q0 = x*r, exact negated
// remainder e = q0*s - x (one fma), corrected quotient q0 - e*r (one fma).
// Using the negated remainder keeps the sign of zero: for x = -0 it yields
// -0 (the plain form q0 + (x - q0*s)*r would give +0).  The result equals the
// IEEE quotient bit for bit wherever |x/s| >= 2^-10; below that both encode
// to a zero of the same sign (checked exhaustively by bs_diag_division).
__device__ __forceinline__ float div_by_scale(float x, Scale sc) {
    const float q0 = x * sc.r;
    const float e = __builtin_fmaf(q0, sc.s, -x);
    return __builtin_fmaf(-e, sc.r, q0);
}

// Clamp to the finite e4m3 range (the hardware convert turns |y| >= 465
// into NaN; -0 stays -0).  This is the definition's saturating step; the hot
// path does not need it (see encode4).
__device__ __forceinline__ float clamp448(float y) {
    return __builtin_amdgcn_fmed3f(y, -kE4m3Max, kE4m3Max);
}

// Four quotients -> four e4m3 codes in one little-endian word (element 0 in
// the low byte).  v_cvt_pk_fp8_f32 rounds to nearest even, keeps the sign of
// zero, and maps every |y| <= 464 into the finite codes (|y| in (448, 464]
// -> +-448).  A quantizer quotient never exceeds 448 * (1 + 2^-23) in
// magnitude (|x| <= max(amax, EPS) and s is that over 448, correctly
// rounded), so no clamp is needed: bs_diag_division checks the codes of this
// routine against the clamped IEEE reference on every reachable pair, and
// bs_diag_e4m3_census checks the convert itself on all |y| <= 464.
__device__ __forceinline__ uint32_t encode4(float y0, float y1, float y2, float y3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
    return (uint32_t)w;
}

// The definition's encode (clamp, then round): the diagnostics' reference.
__device__ __forceinline__ uint32_t encode_clamped(float y) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(y), 0.f, 0, false) & 0xffu;
}

// Unpack a 16-byte chunk of 8 bf16 values to floats.
__device__ __forceinline__ void unpack8(uint4 v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Quantize 8 floats with one scale -> 8 codes (element 0 in the low byte).
__device__ __forceinline__ uint2 quant8(const float* f, Scale sc) {
    uint2 out;
    out.x = encode4(div_by_scale(f[0], sc), div_by_scale(f[1], sc),
                    div_by_scale(f[2], sc), div_by_scale(f[3], sc));
    out.y = encode4(div_by_scale(f[4], sc), div_by_scale(f[5], sc),
                    div_by_scale(f[6], sc), div_by_scale(f[7], sc));
    return out;
}

// DPP max over the 16 lanes of a row (all lanes receive the result).
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));  // row_ror 4
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));  // row_ror 8
    return v;
}

}  // namespace bs
