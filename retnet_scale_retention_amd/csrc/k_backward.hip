// k_backward.hip -- element-wise kernels of the backward pass (gradients of
// the outputs and the outgoing state with respect to Q, K, V and the
// incoming state).  The retention products themselves run on the forward
// kernels: with G = dL/dO_raw, the gradients are three retention calls
// (jsqmd.com "From RoPE to Retention" s4.1 parallel form, differentiated),
//   dq~ = Ret(queries G, keys V, values K~, state S_in^T)            forward in time
//   dk~ = Ret(queries V, keys G, values Q~, state dS_out^T / gamma)  backward in time
//   dV  = Ret(queries K~, keys Q~, values G, state dS_out / gamma)   backward in time
// whose last one also yields dS_in = gamma * (its outgoing state).  Here:
// dtype conversion, rotation to token-major fp32 and its inverse, GroupNorm's
// backward, time reversal, and the state transposes and per-head scalings.
// Tensors are token-major [B][T][H][d]; states [B][H][d1][d2].
#include "msr_device.hpp"

namespace {

using namespace msr;

// N contiguous elements (N = 1, 2, 4, 8; the address aligned to N elements)
// to and from fp32, as one or two vector memory operations
template <int N>
__device__ __forceinline__ void ldv(const uint16_t *p, float (&v)[N]) {
    typedef uint16_t V __attribute__((ext_vector_type(N)));
    const V x = *reinterpret_cast<const V *>(p);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = bf16_to_f32(x[i]);
}
template <int N>
__device__ __forceinline__ void ldv(const float *p, float (&v)[N]) {
    constexpr int M = N > 4 ? 4 : N;
    typedef float V __attribute__((ext_vector_type(M)));
#pragma unroll
    for (int h = 0; h < N / M; ++h) {
        const V x = *reinterpret_cast<const V *>(p + M * h);
#pragma unroll
        for (int i = 0; i < M; ++i) v[M * h + i] = x[i];
    }
}
template <int N>
__device__ __forceinline__ void stv(uint16_t *p, const float (&v)[N]) {
    typedef uint16_t V __attribute__((ext_vector_type(N)));
    V x;
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = f32_to_bf16(v[i]);
    *reinterpret_cast<V *>(p) = x;
}
template <int N>
__device__ __forceinline__ void stv(float *p, const float (&v)[N]) {
    constexpr int M = N > 4 ? 4 : N;
    typedef float V __attribute__((ext_vector_type(M)));
#pragma unroll
    for (int h = 0; h < N / M; ++h) {
        V x;
#pragma unroll
        for (int i = 0; i < M; ++i) x[i] = v[M * h + i];
        *reinterpret_cast<V *>(p + M * h) = x;
    }
}


template <typename TIn>
__global__ void to_f32_kernel(size_t n, const TIn *__restrict__ x, float *__restrict__ y) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
        y[e] = load(x, e);
}

// y = factor * R(+-angle) x per channel pair of each [B][T][H][dk] row;
// sign = +1: the forward rotation, -1: its inverse (the transpose).  TOut is
// the destination element type.  With ylo (bf16 destinations only), y gets
// the bf16 rounding of each fp32 value and ylo the bf16 rounding of what
// that leaves: y + ylo carries about 16 significant bits.
template <typename TIn, typename TOut>
__global__ void rotate_tok_kernel(MsrConst c, const TIn *__restrict__ x, TOut *__restrict__ y,
                                  TOut *__restrict__ ylo, float factor, float sign) {
    const int half = c.dk / 2;
    const size_t n = (size_t)c.B * c.T * c.H * half;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int i = (int)(e % half);
        const size_t r = e / half;  // (b T + t) H + h
        const int t = (int)((r / c.H) % c.T), b = (int)(r / ((size_t)c.H * c.T));
        const float x0 = load(x, 2 * e), x1 = load(x, 2 * e + 1);
        float cs = 1.f, sn = 0.f;
        if (!(c.flags & MSR_FLAG_NO_ROTATE)) rot_cos_sin(row_pos0(c, b) + t, c.theta[i], cs, sn);
        sn *= sign;
        const float a = (x0 * cs - x1 * sn) * factor, b2 = (x1 * cs + x0 * sn) * factor;
        store(y, 2 * e, a);
        store(y, 2 * e + 1, b2);
        if constexpr (sizeof(TOut) == 2) {
            if (ylo) {
                store(ylo, 2 * e, a - bf16_to_f32(f32_to_bf16(a)));
                store(ylo, 2 * e + 1, b2 - bf16_to_f32(f32_to_bf16(b2)));
            }
        }
    }
}

// The same, four pairs (8 elements, one or two 16-byte accesses) per work
// item; d_k a multiple of 8.  rev: output token t reads input token T-1-t of
// its batch row (the rotation still takes the output's position).  x2 (bf16,
// optional, same layout as x) is added to x before the rotation.
template <typename TIn, typename TOut>
__global__ void rotate_tok8_kernel(MsrConst c, const TIn *__restrict__ x, TOut *__restrict__ y,
                                   TOut *__restrict__ ylo, float factor, float sign, int rev,
                                   const uint16_t *__restrict__ x2) {
    const int g8 = c.dk / 8;
    const size_t n = (size_t)c.B * c.T * c.H * g8;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int i0 = (int)(e % g8) * 4;  // first pair
        const size_t r = e / g8;           // (b T + t) H + h
        const int t = (int)((r / c.H) % c.T), b = (int)(r / ((size_t)c.H * c.T));
        float v[8], hi[8], lo[8];
        const size_t rx = rev ? ((size_t)b * c.T + (c.T - 1 - t)) * c.H + r % c.H : r;
        ldv<8>(x + 8 * (rx * g8 + e % g8), v);
        if (x2) {
            float v2[8];
            ldv<8>(x2 + 8 * (rx * g8 + e % g8), v2);
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] += v2[j];
        }
        const bool rot = !(c.flags & MSR_FLAG_NO_ROTATE);
        const int64_t pos = rot ? row_pos0(c, b) + t : 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float cs = 1.f, sn = 0.f;
            if (rot) rot_cos_sin(pos, c.theta[i0 + q], cs, sn);
            sn *= sign;
            const float x0 = v[2 * q], x1 = v[2 * q + 1];
            hi[2 * q] = (x0 * cs - x1 * sn) * factor;
            hi[2 * q + 1] = (x1 * cs + x0 * sn) * factor;
        }
        if constexpr (sizeof(TOut) == 2) {
            if (ylo) {
#pragma unroll
                for (int j = 0; j < 8; ++j) lo[j] = hi[j] - bf16_to_f32(f32_to_bf16(hi[j]));
                stv<8>(ylo + 8 * e, lo);
            }
        }
        stv<8>(y + 8 * e, hi);
    }
}

// GroupNorm backward, one wave per (token, head) row of d_v values:
//   y = (x - mean) s,  s = 1/sqrt(var + eps),
//   dx = s (dy - mean(dy) - y mean(dy y))
template <typename TX, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void gn_backward_kernel(size_t rows, int dv, float eps,
                                                          const TX *__restrict__ x, const TIn *__restrict__ dy,
                                                          TOut *__restrict__ dx) {
    const int lane = threadIdx.x & 63;
    const size_t row = blockIdx.x * (size_t)(blockDim.x / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const size_t r0 = row * dv;
    float s = 0.f;
    for (int j = lane; j < dv; j += 64) s += load(x, r0 + j);
    const float mean = wave_sum(s) / dv;
    float q2 = 0.f;
    for (int j = lane; j < dv; j += 64) {
        const float d = load(x, r0 + j) - mean;
        q2 += d * d;
    }
    const float inv = 1.f / sqrtf(wave_sum(q2) / dv + eps);
    auto yval = [&](int j) { return (load(x, r0 + j) - mean) * inv; };
    float sd = 0.f, sdy = 0.f;
    for (int j = lane; j < dv; j += 64) {
        const float g = load(dy, r0 + j);
        sd += g;
        sdy += g * yval(j);
    }
    const float md = wave_sum(sd) / dv, mdy = wave_sum(sdy) / dv;
    for (int j = lane; j < dv; j += 64) store(dx, r0 + j, inv * (load(dy, r0 + j) - md - yval(j) * mdy));
}

// The same with the row held in registers: lane l owns elements
// [PER l, PER l + PER) of a row of 64 PER values, read and written once.
template <int PER, typename TX, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void gn_backward_row_kernel(size_t rows, float eps, const TX *__restrict__ x,
                                                              const TIn *__restrict__ dy, TOut *__restrict__ dx) {
    constexpr int dv = 64 * PER;
    const int lane = threadIdx.x & 63;
    const size_t row = blockIdx.x * (size_t)(blockDim.x / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const size_t r0 = row * dv + (size_t)PER * lane;
    float xv[PER], gv[PER];
    ldv<PER>(x + r0, xv);
    ldv<PER>(dy + r0, gv);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) s += xv[i];
    const float mean = wave_sum(s) / dv;
    float q2 = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        xv[i] -= mean;
        q2 += xv[i] * xv[i];
    }
    const float inv = 1.f / sqrtf(wave_sum(q2) / dv + eps);
    float sd = 0.f, sdy = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        xv[i] *= inv;  // y
        sd += gv[i];
        sdy += gv[i] * xv[i];
    }
    const float md = wave_sum(sd) / dv, mdy = wave_sum(sdy) / dv;
#pragma unroll
    for (int i = 0; i < PER; ++i) gv[i] = inv * (gv[i] - md - xv[i] * mdy);
    stv<PER>(dx + r0, gv);
}

// y[b][t'][h][0:len] = x[b][t][h][col0:col0+len] with t' = T-1-t when
// reversing, else t: time reversal, a column slice, and dtype conversion
template <typename TIn, typename TOut>
__global__ void slice_kernel(int B, int T, int H, int d, int col0, int len, int reverse, const TIn *__restrict__ x,
                             TOut *__restrict__ y) {
    const size_t n = (size_t)B * T * H * len;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int j = (int)(e % len);
        const size_t r = e / len;  // (b T + t) H + h
        const int h = (int)(r % H);
        const size_t bt = r / H;
        const int t = (int)(bt % T);
        const size_t b = bt / T;
        const size_t src = ((b * T + t) * H + h) * (size_t)d + col0 + j;
        const size_t dst = ((b * T + (reverse ? T - 1 - t : t)) * H + h) * (size_t)len + j;
        store(y, dst, load(x, src));
    }
}

// The same, 8 consecutive elements per work item (d, col0, len multiples of 8)
template <typename TIn, typename TOut>
__global__ void slice8_kernel(int B, int T, int H, int d, int col0, int len, int reverse, const TIn *__restrict__ x,
                              TOut *__restrict__ y) {
    const int l8 = len / 8;
    const size_t n = (size_t)B * T * H * l8;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int j = (int)(e % l8) * 8;
        const size_t r = e / l8;  // (b T + t) H + h
        const int h = (int)(r % H);
        const size_t bt = r / H;
        const int t = (int)(bt % T);
        const size_t b = bt / T;
        float v[8];
        ldv<8>(x + ((b * T + t) * H + h) * (size_t)d + col0 + j, v);
        stv<8>(y + ((b * T + (reverse ? T - 1 - t : t)) * H + h) * (size_t)len + j, v);
    }
}

// y (fp32) = x + (first ? 0 : y)
template <typename TIn>
__global__ void accumulate_kernel(size_t n, const TIn *__restrict__ x, float *__restrict__ y, int first) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
        y[e] = load(x, e) + (first ? 0.f : y[e]);
}

// the same, 8 elements per work item (n a multiple of 8)
template <typename TIn>
__global__ void accumulate8_kernel(size_t n8, const TIn *__restrict__ x, float *__restrict__ y, int first) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n8; e += (size_t)gridDim.x * blockDim.x) {
        float a[8], b[8];
        ldv<8>(x + 8 * e, a);
        if (!first) {
            ldv<8>(y + 8 * e, b);
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] += b[i];
        }
        stv<8>(y + 8 * e, a);
    }
}

// Rows [B][T][H][d] times the row-normalised-decay factor at their absolute
// positions (1 when the problem does not ask for it); y may be x
template <typename TIn, typename TOut>
__global__ void row_scale_kernel(MsrConst c, int d, const TIn *x, TOut *y) {
    const size_t n = (size_t)c.B * c.T * c.H * d;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const size_t r = e / d;  // (b T + t) H + h
        const int h = (int)(r % c.H), t = (int)((r / c.H) % c.T), b = (int)(r / ((size_t)c.H * c.T));
        store(y, e, load(x, e) * row_norm_factor(c, row_pos0(c, b) + t, c.log2g[h]));
    }
}

// States in [B H][d1][d2], f_h = gamma_h^power, in NULL reads as zeros:
//   transpose = 0: out[p][i][j] = f_h in[p][i][j]
//   transpose = 1: out[p][j - j0][i] = f_h in[p][i][j] for j in [j0, j0 + nj)
//                  (a row block of the transpose, [nj][d1] per pair)
__global__ void state_kernel(MsrConst c, int d1, int d2, const float *__restrict__ in, float *__restrict__ out,
                             int transpose, float power, int j0, int nj) {
    const size_t per_out = (size_t)d1 * (transpose ? nj : d2), n = (size_t)c.B * c.H * per_out;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const size_t p = e / per_out, w = e % per_out;
        int i, j;
        if (transpose) {
            j = j0 + (int)(w / d1);
            i = (int)(w % d1);
        } else {
            i = (int)(w / d2);
            j = (int)(w % d2);
        }
        const float f = exp2f(power * c.log2g[p % c.H]);
        out[e] = in ? in[(p * d1 + i) * (size_t)d2 + j] * f : 0.f;
    }
}

unsigned grid_for(size_t n) {
    size_t g = (n + 255) / 256;
    if (g > 65536u) g = 65536u;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_to_f32(int dtype, size_t n, const void *x, float *y, hipStream_t st) {
    if (n == 0) return hipSuccess;
    if (dtype == MSR_BF16)
        hipLaunchKernelGGL(to_f32_kernel<uint16_t>, dim3(grid_for(n)), dim3(256), 0, st, n,
                           static_cast<const uint16_t *>(x), y);
    else
        hipLaunchKernelGGL(to_f32_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, n,
                           static_cast<const float *>(x), y);
    return hipGetLastError();
}

template <typename TIn>
hipError_t rotate_tok_in(const MsrConst &c, const TIn *x, void *y, void *ylo, int out_dtype, float factor,
                         float sign, int rev, const uint16_t *x2, hipStream_t st) {
    const size_t n = (size_t)c.B * c.T * c.H * (c.dk / 2);
    if (n == 0) return hipSuccess;
    if ((rev || x2) && c.dk % 8 != 0) return hipErrorNotSupported;
    if (c.dk % 8 == 0) {
        const size_t n8 = n / 4;
        if (out_dtype == MSR_BF16)
            hipLaunchKernelGGL((rotate_tok8_kernel<TIn, uint16_t>), dim3(grid_for(n8)), dim3(256), 0, st, c, x,
                               static_cast<uint16_t *>(y), static_cast<uint16_t *>(ylo), factor, sign, rev, x2);
        else
            hipLaunchKernelGGL((rotate_tok8_kernel<TIn, float>), dim3(grid_for(n8)), dim3(256), 0, st, c, x,
                               static_cast<float *>(y), nullptr, factor, sign, rev, x2);
        return hipGetLastError();
    }
    if (out_dtype == MSR_BF16)
        hipLaunchKernelGGL((rotate_tok_kernel<TIn, uint16_t>), dim3(grid_for(n)), dim3(256), 0, st, c, x,
                           static_cast<uint16_t *>(y), static_cast<uint16_t *>(ylo), factor, sign);
    else
        hipLaunchKernelGGL((rotate_tok_kernel<TIn, float>), dim3(grid_for(n)), dim3(256), 0, st, c, x,
                           static_cast<float *>(y), nullptr, factor, sign);
    return hipGetLastError();
}

hipError_t launch_rotate_tok(const MsrConst &c, const void *x, int in_dtype, void *y, int out_dtype, float factor,
                             float sign, hipStream_t st, void *ylo, int rev, const void *x2) {
    if (ylo && out_dtype != MSR_BF16) return hipErrorInvalidValue;
    const uint16_t *a2 = static_cast<const uint16_t *>(x2);
    if (in_dtype == MSR_BF16)
        return rotate_tok_in(c, static_cast<const uint16_t *>(x), y, ylo, out_dtype, factor, sign, rev, a2, st);
    return rotate_tok_in(c, static_cast<const float *>(x), y, ylo, out_dtype, factor, sign, rev, a2, st);
}

template <int PER, typename TX, typename TIn>
hipError_t gn_backward_row(size_t rows, float eps, const TX *x, const TIn *dy, void *dx, int out_dtype,
                           hipStream_t st) {
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    if (out_dtype == MSR_BF16)
        hipLaunchKernelGGL((gn_backward_row_kernel<PER, TX, TIn, uint16_t>), dim3(blocks), dim3(256), 0, st, rows,
                           eps, x, dy, static_cast<uint16_t *>(dx));
    else
        hipLaunchKernelGGL((gn_backward_row_kernel<PER, TX, TIn, float>), dim3(blocks), dim3(256), 0, st, rows, eps,
                           x, dy, static_cast<float *>(dx));
    return hipGetLastError();
}

template <typename TX, typename TIn>
hipError_t gn_backward_in(size_t rows, int dv, float eps, const TX *x, const TIn *dy, void *dx, int out_dtype,
                          hipStream_t st) {
    switch (dv) {  // rows of 64, 128, 256, 512 values: held in registers
        case 64: return gn_backward_row<1>(rows, eps, x, dy, dx, out_dtype, st);
        case 128: return gn_backward_row<2>(rows, eps, x, dy, dx, out_dtype, st);
        case 256: return gn_backward_row<4>(rows, eps, x, dy, dx, out_dtype, st);
        case 512: return gn_backward_row<8>(rows, eps, x, dy, dx, out_dtype, st);
        default: break;
    }
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    if (out_dtype == MSR_BF16)
        hipLaunchKernelGGL((gn_backward_kernel<TX, TIn, uint16_t>), dim3(blocks), dim3(256), 0, st, rows, dv, eps, x,
                           dy, static_cast<uint16_t *>(dx));
    else
        hipLaunchKernelGGL((gn_backward_kernel<TX, TIn, float>), dim3(blocks), dim3(256), 0, st, rows, dv, eps, x,
                           dy, static_cast<float *>(dx));
    return hipGetLastError();
}

hipError_t launch_gn_backward(size_t rows, int dv, float eps, const void *x, int x_dtype, const void *dy,
                              int dy_dtype, void *dx, int out_dtype, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const bool xb = x_dtype == MSR_BF16, yb = dy_dtype == MSR_BF16;
    typedef const uint16_t *HB;
    typedef const float *HF;
    if (xb && yb) return gn_backward_in(rows, dv, eps, HB(x), HB(dy), dx, out_dtype, st);
    if (xb) return gn_backward_in(rows, dv, eps, HB(x), HF(dy), dx, out_dtype, st);
    if (yb) return gn_backward_in(rows, dv, eps, HF(x), HB(dy), dx, out_dtype, st);
    return gn_backward_in(rows, dv, eps, HF(x), HF(dy), dx, out_dtype, st);
}

template <typename TIn>
hipError_t slice_in(int B, int T, int H, int d, int col0, int len, int reverse, const TIn *x, void *y, int out_dtype,
                    hipStream_t st) {
    const size_t n = (size_t)B * T * H * len;
    if (n == 0) return hipSuccess;
    if (d % 8 == 0 && col0 % 8 == 0 && len % 8 == 0) {
        if (out_dtype == MSR_BF16)
            hipLaunchKernelGGL((slice8_kernel<TIn, uint16_t>), dim3(grid_for(n / 8)), dim3(256), 0, st, B, T, H, d,
                               col0, len, reverse, x, static_cast<uint16_t *>(y));
        else
            hipLaunchKernelGGL((slice8_kernel<TIn, float>), dim3(grid_for(n / 8)), dim3(256), 0, st, B, T, H, d,
                               col0, len, reverse, x, static_cast<float *>(y));
        return hipGetLastError();
    }
    if (out_dtype == MSR_BF16)
        hipLaunchKernelGGL((slice_kernel<TIn, uint16_t>), dim3(grid_for(n)), dim3(256), 0, st, B, T, H, d, col0, len,
                           reverse, x, static_cast<uint16_t *>(y));
    else
        hipLaunchKernelGGL((slice_kernel<TIn, float>), dim3(grid_for(n)), dim3(256), 0, st, B, T, H, d, col0, len,
                           reverse, x, static_cast<float *>(y));
    return hipGetLastError();
}

hipError_t launch_slice(int B, int T, int H, int d, int col0, int len, int reverse, const void *x, int in_dtype,
                        void *y, int out_dtype, hipStream_t st) {
    if (in_dtype == MSR_BF16)
        return slice_in(B, T, H, d, col0, len, reverse, static_cast<const uint16_t *>(x), y, out_dtype, st);
    return slice_in(B, T, H, d, col0, len, reverse, static_cast<const float *>(x), y, out_dtype, st);
}

hipError_t launch_row_scale(const MsrConst &c, int d, const void *x, int in_dtype, void *y, int out_dtype,
                            hipStream_t st) {
    const size_t n = (size_t)c.B * c.T * c.H * d;
    if (n == 0) return hipSuccess;
    typedef const uint16_t *HB;
    typedef const float *HF;
    typedef uint16_t *OB;
    typedef float *OF;
    if (in_dtype == MSR_BF16 && out_dtype == MSR_BF16)
        hipLaunchKernelGGL((row_scale_kernel<uint16_t, uint16_t>), dim3(grid_for(n)), dim3(256), 0, st, c, d, HB(x), OB(y));
    else if (in_dtype == MSR_BF16)
        hipLaunchKernelGGL((row_scale_kernel<uint16_t, float>), dim3(grid_for(n)), dim3(256), 0, st, c, d, HB(x), OF(y));
    else if (out_dtype == MSR_BF16)
        hipLaunchKernelGGL((row_scale_kernel<float, uint16_t>), dim3(grid_for(n)), dim3(256), 0, st, c, d, HF(x), OB(y));
    else
        hipLaunchKernelGGL((row_scale_kernel<float, float>), dim3(grid_for(n)), dim3(256), 0, st, c, d, HF(x), OF(y));
    return hipGetLastError();
}

hipError_t launch_accumulate(size_t n, const void *x, int in_dtype, float *y, int first, hipStream_t st) {
    if (n == 0) return hipSuccess;
    if (n % 8 == 0) {
        if (in_dtype == MSR_BF16)
            hipLaunchKernelGGL(accumulate8_kernel<uint16_t>, dim3(grid_for(n / 8)), dim3(256), 0, st, n / 8,
                               static_cast<const uint16_t *>(x), y, first);
        else
            hipLaunchKernelGGL(accumulate8_kernel<float>, dim3(grid_for(n / 8)), dim3(256), 0, st, n / 8,
                               static_cast<const float *>(x), y, first);
        return hipGetLastError();
    }
    if (in_dtype == MSR_BF16)
        hipLaunchKernelGGL(accumulate_kernel<uint16_t>, dim3(grid_for(n)), dim3(256), 0, st, n,
                           static_cast<const uint16_t *>(x), y, first);
    else
        hipLaunchKernelGGL(accumulate_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, n,
                           static_cast<const float *>(x), y, first);
    return hipGetLastError();
}

hipError_t launch_state_op(const MsrConst &c, int d1, int d2, const float *in, float *out, int transpose,
                           float power, int j0, int nj, hipStream_t st) {
    const size_t n = (size_t)c.B * c.H * d1 * (transpose ? nj : d2);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(state_kernel, dim3(grid_for(n)), dim3(256), 0, st, c, d1, d2, in, out, transpose, power, j0,
                       nj);
    return hipGetLastError();
}
