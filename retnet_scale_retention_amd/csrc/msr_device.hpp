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
// cos and sin of the rotation angle pos * theta.  The angle in quarter
// turns, pos * theta * 2/pi, is formed in fp64 (pos reaches 1e5 and more,
// where an fp32 product would already be off by ~1e-2 rad) and split into
// the nearest whole number q and a remainder in [-1/2, 1/2] (exact: the
// subtraction of q loses no bits); sin and cos of the remainder
// y in [-pi/4, pi/4] radians come from their Taylor series up to y^9 and
// y^10 (truncation below 2e-9 and 1.2e-10), and q mod 4 quarter turns then
// rotate the pair.
__device__ __forceinline__ void rot_cos_sin(int64_t pos, float theta, float &cs, float &sn) {
    const double qt = static_cast<double>(pos) * (static_cast<double>(theta) * 0.63661977236758134);  // 2 / pi
    const double q = rint(qt);
    const float y = static_cast<float>(qt - q) * 1.57079633f;
    const float y2 = y * y;
    const float s = y * (1.f - y2 * (1.f / 6.f - y2 * (1.f / 120.f - y2 * (1.f / 5040.f - y2 * (1.f / 362880.f)))));
    const float c =
        1.f - y2 * (0.5f - y2 * (1.f / 24.f - y2 * (1.f / 720.f - y2 * (1.f / 40320.f - y2 * (1.f / 3628800.f)))));
    // (c, s) turned by qq quarter turns: (c, s), (-s, c), (-c, -s), (s, -c)
    const int qq = static_cast<int>(q - 4.0 * floor(q * 0.25));
    const float a = (qq & 1) ? s : c, b = (qq & 1) ? c : s;
    cs = (qq == 1 || qq == 2) ? -a : a;
    sn = (qq >= 2) ? -b : b;
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

// ---- segmented chunk recurrence -------------------------------------------
// Folds the end states E_0 .. E_(seg-1) of a pair's earlier segments into
// the state tiles (4-float vectors V4) a lane holds, in segment order: S <- S gseg + E_g.  The
// loads do not depend on S, so SB segments' tiles are loaded together and
// folded afterwards: one memory round trip per SB segments instead of one
// per segment (SB sized so the batch takes at most REGS registers).
// off(rt, ct, r) is the element's offset within a segment's state, estride
// the distance between segments.
template <int REGS, int RPW, int CPW, class V4, class Off>
__device__ __forceinline__ void fold_segments(V4 (&S)[RPW][CPW], const float *e0, size_t estride, int seg,
                                              float gseg, Off off) {
    constexpr int SB = 4 * RPW * CPW >= REGS ? 1 : REGS / (4 * RPW * CPW);
    if constexpr (SB == 1) {
        // no room for a staged batch: each load feeds its own fold
        for (int gg = 0; gg < seg; ++gg) {
            const float *e = e0 + (size_t)gg * estride;
#pragma unroll
            for (int rt = 0; rt < RPW; ++rt)
#pragma unroll
                for (int ct = 0; ct < CPW; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[rt][ct][r] = S[rt][ct][r] * gseg + e[off(rt, ct, r)];
        }
        return;
    }
    for (int g0 = 0; g0 < seg; g0 += SB) {
        V4 ev[SB][RPW][CPW];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            // past the last segment: a repeat of it, loaded but not folded
            const float *e = e0 + (size_t)(g0 + u < seg ? g0 + u : seg - 1) * estride;
#pragma unroll
            for (int rt = 0; rt < RPW; ++rt)
#pragma unroll
                for (int ct = 0; ct < CPW; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) ev[u][rt][ct][r] = e[off(rt, ct, r)];
        }
#pragma unroll
        for (int u = 0; u < SB; ++u)
            if (g0 + u < seg) {
#pragma unroll
                for (int rt = 0; rt < RPW; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CPW; ++ct) S[rt][ct] = S[rt][ct] * gseg + ev[u][rt][ct];
            }
    }
}

}  // namespace msr
