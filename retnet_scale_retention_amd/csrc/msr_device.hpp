// msr_device.hpp -- device-side helpers shared by the HIP kernels:
// bf16 <-> fp32 conversion, the rotation angle, the decay weight and
// block-wide reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msr_internal.hpp"

namespace msr {

// ---- element access: fp32 tensors are float, bf16 tensors are raw uint16 --
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float load(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float load(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void store(float *p, size_t i, float x) { p[i] = x; }
__device__ __forceinline__ void store(uint16_t *p, size_t i, float x) { p[i] = f32_to_bf16(x); }

// ---- rotation angle ---------------------------------------------------------
// cos/sin of pos * theta.  The product and the reduction modulo 2*pi are done
// in fp64 (pos reaches 1e5 and more, where an fp32 product would already be
// off by ~1e-2 rad); the reduced angle in [-pi, pi] is then evaluated in fp32.
// 2*pi is split in two doubles (Cody and Waite's argument reduction).
__device__ __forceinline__ void rot_cos_sin(int64_t pos, float theta, float &cs, float &sn) {
    const double two_pi_hi = 6.283185307179586;       // nearest double to 2*pi
    const double two_pi_lo = 2.4492935982947064e-16;  // 2*pi - two_pi_hi
    const double inv_two_pi = 0.15915494309189535;
    double phi = static_cast<double>(pos) * static_cast<double>(theta);
    double k = rint(phi * inv_two_pi);
    double r = fma(-k, two_pi_hi, phi);
    r = fma(-k, two_pi_lo, r);
    sincosf(static_cast<float>(r), &sn, &cs);
}

// position of token 0 of batch row b
__device__ __forceinline__ int64_t row_pos0(const MsrConst &c, int b) { return c.pos_rows ? c.pos_rows[b] : c.pos0; }

// Sum of the decay weights of the row at absolute position p,
// sum_{j=0}^{p} gamma^j = (1 - gamma^(p+1)) / (1 - gamma), formed as a ratio
// of expm1 values so that gamma near 1 keeps its relative accuracy; p + 1
// when gamma = 1.
__device__ __forceinline__ float decay_row_sum(int64_t p, float log2g) {
    if (log2g == 0.f) return (float)(p + 1);
    const float l = log2g * 0.693147180559945f;
    return expm1f((float)(p + 1) * l) / expm1f(l);
}

// 1 / decay_row_sum when the problem asks for row-normalised decay, else 1
__device__ __forceinline__ float row_norm_factor(const MsrConst &c, int64_t p, float log2g) {
    return (c.flags & MSR_FLAG_DECAY_ROWNORM) ? 1.f / decay_row_sum(p, log2g) : 1.f;
}

// gamma^d for d >= 0, as 2^(d * log2 gamma); never forms gamma^(-d).
__device__ __forceinline__ float decay(float d, float log2g) { return exp2f(d * log2g); }

// ---- reductions ---------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Sum over the whole block; `red` holds one float per wave (<= 16 waves).
// Every thread of the block must call it; all get the result.
__device__ __forceinline__ float block_sum(float x, float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    x = wave_sum(x);
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[w];
    return s;
}

}  // namespace msr
