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


template <typename TIn>
__global__ void to_f32_kernel(size_t n, const TIn *__restrict__ x, float *__restrict__ y) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
        y[e] = load(x, e);
}

// y = factor * R(+-angle) x per channel pair of each [B][T][H][dk] row;
// sign = +1: the forward rotation, -1: its inverse (the transpose).  TOut is
// the destination element type.
template <typename TOut>
__global__ void rotate_tok_kernel(MsrConst c, const float *__restrict__ x, TOut *__restrict__ y, float factor,
                                  float sign) {
    const int half = c.dk / 2;
    const size_t n = (size_t)c.B * c.T * c.H * half;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int i = (int)(e % half);
        const size_t r = e / half;  // (b T + t) H + h
        const int t = (int)((r / c.H) % c.T), b = (int)(r / ((size_t)c.H * c.T));
        const float x0 = x[2 * e], x1 = x[2 * e + 1];
        float cs = 1.f, sn = 0.f;
        if (!(c.flags & MSR_FLAG_NO_ROTATE)) rot_cos_sin(row_pos0(c, b) + t, c.theta[i], cs, sn);
        sn *= sign;
        store(y, 2 * e, (x0 * cs - x1 * sn) * factor);
        store(y, 2 * e + 1, (x1 * cs + x0 * sn) * factor);
    }
}

// GroupNorm backward, one wave per (token, head) row of d_v values:
//   y = (x - mean) s,  s = 1/sqrt(var + eps),
//   dx = s (dy - mean(dy) - y mean(dy y))
template <typename TIn>
__global__ __launch_bounds__(256) void gn_backward_kernel(size_t rows, int dv, float eps,
                                                          const float *__restrict__ x,
                                                          const TIn *__restrict__ dy, float *__restrict__ dx) {
    const int lane = threadIdx.x & 63;
    const size_t row = blockIdx.x * (size_t)(blockDim.x / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *xr = x + row * dv;
    float s = 0.f;
    for (int j = lane; j < dv; j += 64) s += xr[j];
    const float mean = wave_sum(s) / dv;
    float q2 = 0.f;
    for (int j = lane; j < dv; j += 64) q2 += (xr[j] - mean) * (xr[j] - mean);
    const float inv = 1.f / sqrtf(wave_sum(q2) / dv + eps);
    float sd = 0.f, sdy = 0.f;
    for (int j = lane; j < dv; j += 64) {
        const float g = load(dy, row * dv + j);
        sd += g;
        sdy += g * (xr[j] - mean) * inv;
    }
    const float md = wave_sum(sd) / dv, mdy = wave_sum(sdy) / dv;
    for (int j = lane; j < dv; j += 64) {
        const float yv = (xr[j] - mean) * inv;
        dx[row * dv + j] = inv * (load(dy, row * dv + j) - md - yv * mdy);
    }
}

// y[b][T-1-t][h][:] = x[b][t][h][:] (element type of y: TOut)
template <typename TOut>
__global__ void reverse_kernel(int B, int T, int H, int d, const float *__restrict__ x, TOut *__restrict__ y) {
    const size_t row = (size_t)H * d, n = (size_t)B * T * row;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const size_t bt = e / row, w = e % row;
        const int t = (int)(bt % T);
        const size_t b = bt / T;
        store(y, (b * T + (T - 1 - t)) * row + w, x[e]);
    }
}

// out[p][j][i] = f_h * in[p][i][j] (transpose = 1) or out[p][i][j] = f_h *
// in[p][i][j] (transpose = 0), f_h = gamma_h^power; in NULL gives zeros
__global__ void state_kernel(MsrConst c, int d1, int d2, const float *__restrict__ in, float *__restrict__ out,
                             int transpose, float power) {
    const size_t per = (size_t)d1 * d2, n = (size_t)c.B * c.H * per;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const size_t p = e / per, w = e % per;
        const int i = (int)(w / d2), j = (int)(w % d2);
        const float f = exp2f(power * c.log2g[p % c.H]);
        const float v = in ? in[e] * f : 0.f;
        out[p * per + (transpose ? (size_t)j * d1 + i : w)] = v;
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

hipError_t launch_rotate_tok(const MsrConst &c, const float *x, void *y, int out_dtype, float factor, float sign,
                             hipStream_t st) {
    const size_t n = (size_t)c.B * c.T * c.H * (c.dk / 2);
    if (n == 0) return hipSuccess;
    if (out_dtype == MSR_BF16)
        hipLaunchKernelGGL(rotate_tok_kernel<uint16_t>, dim3(grid_for(n)), dim3(256), 0, st, c, x,
                           static_cast<uint16_t *>(y), factor, sign);
    else
        hipLaunchKernelGGL(rotate_tok_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, c, x,
                           static_cast<float *>(y), factor, sign);
    return hipGetLastError();
}

hipError_t launch_gn_backward(int dtype, size_t rows, int dv, float eps, const float *x, const void *dy, float *dx,
                              hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    if (dtype == MSR_BF16)
        hipLaunchKernelGGL(gn_backward_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st, rows, dv, eps, x,
                           static_cast<const uint16_t *>(dy), dx);
    else
        hipLaunchKernelGGL(gn_backward_kernel<float>, dim3(blocks), dim3(256), 0, st, rows, dv, eps, x,
                           static_cast<const float *>(dy), dx);
    return hipGetLastError();
}

hipError_t launch_reverse(int B, int T, int H, int d, const float *x, void *y, int out_dtype, hipStream_t st) {
    const size_t n = (size_t)B * T * H * d;
    if (n == 0) return hipSuccess;
    if (out_dtype == MSR_BF16)
        hipLaunchKernelGGL(reverse_kernel<uint16_t>, dim3(grid_for(n)), dim3(256), 0, st, B, T, H, d, x,
                           static_cast<uint16_t *>(y));
    else
        hipLaunchKernelGGL(reverse_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, B, T, H, d, x,
                           static_cast<float *>(y));
    return hipGetLastError();
}

hipError_t launch_state_op(const MsrConst &c, int d1, int d2, const float *in, float *out, int transpose,
                           float power, hipStream_t st) {
    const size_t n = (size_t)c.B * c.H * d1 * d2;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(state_kernel, dim3(grid_for(n)), dim3(256), 0, st, c, d1, d2, in, out, transpose, power);
    return hipGetLastError();
}
