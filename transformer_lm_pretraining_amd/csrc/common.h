// Shared device helpers for the gfx950 kernels: bf16 conversion, MFMA
// fragment types, wavefront reductions, launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define WAVE 64

// fp32 -> bf16 bits, round to nearest even (the gfx950 conversion instruction,
// v_cvt_pk_bf16_f32, which also keeps NaN a NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Sum / max over the 64 lanes of a wavefront (result in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// 32x32x16 bf16 MFMA: D[i][j] = sum_k A[i][k] B[k][j] + C.  Lane l supplies
// A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32]; the result register r
// of lane l holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Pack 8 floats into 8 bf16 (as an MFMA operand).
__device__ __forceinline__ bf16x8 pack8(const float* f) {
    u32x4 w;
    w.x = pack_bf2(f[0], f[1]);
    w.y = pack_bf2(f[2], f[3]);
    w.z = pack_bf2(f[4], f[5]);
    w.w = pack_bf2(f[6], f[7]);
    return as_bf16x8(w);
}

// Transpose an 8x8 block of bf16 held as 8 rows of 8 (in[r] = row r).  On
// return out[c] holds column c: (in[0][c], in[1][c], ..., in[7][c]).
__device__ __forceinline__ void transpose8x8(const u32x4* in, u32x4* out) {
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {      // column pair (2*c2, 2*c2+1) = dword c2 of each row
        uint32_t w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) w[r] = in[r][c2];
        u32x4 lo, hi;
        // even column: low halves; odd column: high halves
        lo.x = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
        lo.z = __builtin_amdgcn_perm(w[5], w[4], 0x05040100u);
        lo.w = __builtin_amdgcn_perm(w[7], w[6], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
        hi.z = __builtin_amdgcn_perm(w[5], w[4], 0x07060302u);
        hi.w = __builtin_amdgcn_perm(w[7], w[6], 0x07060302u);
        out[2 * c2] = lo;
        out[2 * c2 + 1] = hi;
    }
}

// GPT-2's tanh-form GELU and its derivative, evaluated in fp32.  With
// a = sqrt(2/pi) (x + 0.044715 x^3), 0.5 (1 + tanh(a)) is the logistic sigmoid
// s = 1 / (1 + exp(-2a)), so GELU(x) = x s and GELU'(x) = s + x s (1 - s) da2/dx
// with da2/dx = 2 sqrt(2/pi) (1 + 3 * 0.044715 x^2).  exp(-2a) is taken as the
// hardware base-2 exponential of x (c0 + c1 x^2); where it overflows, s is 0.
__device__ __forceinline__ float gelu_sigmoid(float x, float x2) {
    const float c0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
    const float c1 = c0 * 0.044715f;
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * fmaf(c1, x2, c0)));
}
__device__ __forceinline__ float gelu_f(float x) { return x * gelu_sigmoid(x, x * x); }
__device__ __forceinline__ float gelu_grad_f(float x) {
    const float x2 = x * x;
    const float s = gelu_sigmoid(x, x2);
    const float d = fmaf(2.0f * 0.7978845608028654f * 3.0f * 0.044715f, x2, 2.0f * 0.7978845608028654f);
    return fmaf(x * s * (1.0f - s), d, s);
}
// Both at once (one exponential and one reciprocal).
__device__ __forceinline__ void gelu_and_grad_f(float x, float& g, float& gp) {
    const float x2 = x * x;
    const float s = gelu_sigmoid(x, x2);
    const float d = fmaf(2.0f * 0.7978845608028654f * 3.0f * 0.044715f, x2, 2.0f * 0.7978845608028654f);
    g = x * s;
    gp = fmaf(g * (1.0f - s), d, s);
}

__host__ __device__ static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
