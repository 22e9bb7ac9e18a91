// k_generic.hip -- the generic (SIMT, fp32 arithmetic) path of all three
// forms.  It handles every shape the ABI accepts and both dtypes; it is the
// path for fp32 problems and the fallback for bf16 shapes the MFMA kernels
// do not cover.  Three kernels:
//   rotate_kernel          Q -> Q~ and K -> s K~ (fp32 copies in workspace)
//   generic_state_kernel   chunk states S_i = gamma^b S_{i-1} + K~^T (V . zeta)
//   generic_output_kernel  O = GN( (Q~K~^T . D) V + xi . (Q~ S_{i-1}) )
// (jsqmd.com "From RoPE to Retention" s2-s5; aiqz.cc RetNet tutorial,
// parallel / chunkwise representations.)
#include "msr_device.hpp"

namespace {

using namespace msr;

// One thread per channel pair of one token.
template <typename TIn>
__global__ void rotate_kernel(MsrConst c, const TIn *__restrict__ x, float *__restrict__ xr,
                              float factor) {
    const int half = c.dk / 2;
    const size_t n = static_cast<size_t>(c.B) * c.T * c.H * half;
    for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < n;
         e += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const int i = static_cast<int>(e % half);
        size_t r = e / half;
        const int h = static_cast<int>(r % c.H);
        r /= c.H;
        const int t = static_cast<int>(r % c.T);
        const int b = static_cast<int>(r / c.T);
        const size_t src = ((static_cast<size_t>(b) * c.T + t) * c.H + h) * c.dk + 2 * i;
        const float x0 = load(x, src), x1 = load(x, src + 1);
        float y0 = x0, y1 = x1;
        if (!(c.flags & MSR_FLAG_NO_ROTATE)) {
            float cs, sn;
            rot_cos_sin(row_pos0(c, b) + t, c.theta[i], cs, sn);
            y0 = x0 * cs - x1 * sn;
            y1 = x1 * cs + x0 * sn;
        }
        const size_t dst = ((static_cast<size_t>(b) * c.H + h) * c.T + t) * c.dk + 2 * i;
        xr[dst] = y0 * factor;
        xr[dst + 1] = y1 * factor;
    }
}

// grid (pairs, ceil(dk/16), ceil(dv/16)), block 16x16: each thread owns one
// state element S[i][j] and walks the chunks in order.
template <typename TIn>
__global__ __launch_bounds__(256) void generic_state_kernel(
    MsrConst c, int chunk, const float *__restrict__ kr, const TIn *__restrict__ v,
    const float *s_in, float *s_out, float *__restrict__ chunk_states) {
    const int pair = blockIdx.x, b = pair / c.H, h = pair % c.H;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int i = blockIdx.y * 16 + ty, j = blockIdx.z * 16 + tx;
    const bool valid = i < c.dk && j < c.dv;
    __shared__ float ks[16][17];  // [token][row]
    __shared__ float vs[16][17];  // [token][col]
    const size_t sidx = (static_cast<size_t>(pair) * c.dk + i) * c.dv + j;
    float S = (valid && s_in) ? s_in[sidx] : 0.f;
    const float lg = c.log2g[h];
    // the last chunk holds T - (nchunks - 1) chunk tokens when chunk does not divide T
    const int nchunks = (c.T + chunk - 1) / chunk;
    for (int ci = 0; ci < nchunks; ++ci) {
        if (chunk_states && valid)
            chunk_states[((static_cast<size_t>(pair) * nchunks + ci) * c.dk + i) * c.dv + j] = S;
        const int len = min(chunk, c.T - ci * chunk);
        float acc = 0.f;
        for (int t0 = 0; t0 < len; t0 += 16) {
            const int tl = t0 + ty;
            const size_t tok = static_cast<size_t>(ci) * chunk + tl;
            const int ii = blockIdx.y * 16 + tx, jj = blockIdx.z * 16 + tx;
            ks[ty][tx] = (tl < len && ii < c.dk)
                             ? kr[(static_cast<size_t>(pair) * c.T + tok) * c.dk + ii] : 0.f;
            vs[ty][tx] = (tl < len && jj < c.dv)
                             ? load(v, ((static_cast<size_t>(b) * c.T + tok) * c.H + h) * c.dv + jj)
                             : 0.f;
            __syncthreads();
            const int nt = min(16, len - t0);
            for (int u = 0; u < nt; ++u) {
                const float z = decay(static_cast<float>(len - 1 - (t0 + u)), lg);
                acc += z * ks[u][ty] * vs[u][tx];
            }
            __syncthreads();
        }
        S = decay(static_cast<float>(len), lg) * S + acc;
    }
    if (s_out && valid) s_out[sidx] = S;
}

constexpr int OUT_THREADS = 256;
constexpr int OUT_KEYS = 1024;  // keys scored per pass
constexpr int OUT_COLS = MSR_MAX_DV / OUT_THREADS;

// grid (T, pairs), block 256: one block per (token, pair).
template <typename TIn>
__global__ __launch_bounds__(OUT_THREADS) void generic_output_kernel(
    MsrConst c, int chunk, const float *__restrict__ qr, const float *__restrict__ kr,
    const TIn *__restrict__ v, TIn *__restrict__ o, const float *states, int64_t pair_stride,
    int64_t chunk_stride) {
    const int n = blockIdx.x, pair = blockIdx.y, b = pair / c.H, h = pair % c.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NW = OUT_THREADS / 64;
    __shared__ float qs[MSR_MAX_DK];
    __shared__ float w[OUT_KEYS];
    __shared__ float red[16];
    const float *qrow = qr + (static_cast<size_t>(pair) * c.T + n) * c.dk;
    for (int i = tid; i < c.dk; i += OUT_THREADS) qs[i] = qrow[i];
    __syncthreads();
    const int c0 = (n / chunk) * chunk, jloc = n - c0;
    const float lg = c.log2g[h];
    float acc[OUT_COLS];
#pragma unroll
    for (int r = 0; r < OUT_COLS; ++r) acc[r] = 0.f;
    for (int m0 = c0; m0 <= n; m0 += OUT_KEYS) {
        const int mend = min(n + 1, m0 + OUT_KEYS);
        for (int m = m0 + wave; m < mend; m += NW) {
            const float *krow = kr + (static_cast<size_t>(pair) * c.T + m) * c.dk;
            float d = 0.f;
            for (int i = lane; i < c.dk; i += 64) d += qs[i] * krow[i];
            d = wave_sum(d);
            if (lane == 0) w[m - m0] = d * decay(static_cast<float>(n - m), lg);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < OUT_COLS; ++r) {
            const int col = tid + r * OUT_THREADS;
            if (col < c.dv) {
                float a = acc[r];
                for (int m = m0; m < mend; ++m)
                    a += w[m - m0] * load(v, ((static_cast<size_t>(b) * c.T + m) * c.H + h) * c.dv + col);
                acc[r] = a;
            }
        }
        __syncthreads();
    }
    if (states) {
        const float *S = states + pair * pair_stride + static_cast<int64_t>(n / chunk) * chunk_stride;
        const float xi = decay(static_cast<float>(jloc + 1), lg);
#pragma unroll
        for (int r = 0; r < OUT_COLS; ++r) {
            const int col = tid + r * OUT_THREADS;
            if (col < c.dv) {
                float a = 0.f;
                for (int i = 0; i < c.dk; ++i) a += qs[i] * S[static_cast<size_t>(i) * c.dv + col];
                acc[r] += xi * a;
            }
        }
    }
    if (c.flags & MSR_FLAG_DECAY_ROWNORM) {
        const float f = row_norm_factor(c, row_pos0(c, b) + n, lg);
#pragma unroll
        for (int r = 0; r < OUT_COLS; ++r) acc[r] *= f;
    }
    if (!(c.flags & MSR_FLAG_NO_GROUPNORM)) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < OUT_COLS; ++r)
            if (tid + r * OUT_THREADS < c.dv) s += acc[r];
        const float mean = block_sum(s, red) / c.dv;
        float q2 = 0.f;
#pragma unroll
        for (int r = 0; r < OUT_COLS; ++r)
            if (tid + r * OUT_THREADS < c.dv) q2 += (acc[r] - mean) * (acc[r] - mean);
        const float var = block_sum(q2, red) / c.dv;
        const float inv = 1.f / sqrtf(var + c.eps);
#pragma unroll
        for (int r = 0; r < OUT_COLS; ++r) acc[r] = (acc[r] - mean) * inv;
    }
    const size_t obase = ((static_cast<size_t>(b) * c.T + n) * c.H + h) * c.dv;
#pragma unroll
    for (int r = 0; r < OUT_COLS; ++r) {
        const int col = tid + r * OUT_THREADS;
        if (col < c.dv) store(o, obase + col, acc[r]);
    }
}

__global__ void copy_state_kernel(size_t n, const float *s_in, float *s_out) {
    for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < n;
         e += static_cast<size_t>(gridDim.x) * blockDim.x)
        s_out[e] = s_in ? s_in[e] : 0.f;
}

unsigned grid_for(size_t n, unsigned block) {
    size_t g = (n + block - 1) / block;
    if (g > 65536u) g = 65536u;
    return static_cast<unsigned>(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_rotate(const MsrConst &c, int dtype, const void *X, float *Xr, float factor,
                         hipStream_t st) {
    const size_t n = static_cast<size_t>(c.B) * c.T * c.H * (c.dk / 2);
    if (n == 0) return hipSuccess;
    const unsigned g = grid_for(n, 256);
    if (dtype == MSR_BF16)
        hipLaunchKernelGGL(rotate_kernel<uint16_t>, dim3(g), dim3(256), 0, st, c,
                           static_cast<const uint16_t *>(X), Xr, factor);
    else
        hipLaunchKernelGGL(rotate_kernel<float>, dim3(g), dim3(256), 0, st, c,
                           static_cast<const float *>(X), Xr, factor);
    return hipGetLastError();
}

hipError_t launch_generic_state(const MsrConst &c, int dtype, int chunk, const float *Kr,
                                const void *V, const float *s_in, float *s_out,
                                float *chunk_states, hipStream_t st) {
    const int pairs = c.B * c.H;
    if (pairs == 0) return hipSuccess;
    dim3 grid(pairs, (c.dk + 15) / 16, (c.dv + 15) / 16);
    if (dtype == MSR_BF16)
        hipLaunchKernelGGL(generic_state_kernel<uint16_t>, grid, dim3(256), 0, st, c, chunk, Kr,
                           static_cast<const uint16_t *>(V), s_in, s_out, chunk_states);
    else
        hipLaunchKernelGGL(generic_state_kernel<float>, grid, dim3(256), 0, st, c, chunk, Kr,
                           static_cast<const float *>(V), s_in, s_out, chunk_states);
    return hipGetLastError();
}

hipError_t launch_generic_output(const MsrConst &c, int dtype, int chunk, const float *Qr,
                                 const float *Kr, const void *V, void *O, const float *states,
                                 int64_t pair_stride, int64_t chunk_stride, hipStream_t st) {
    const int pairs = c.B * c.H;
    if (pairs == 0 || c.T == 0) return hipSuccess;
    dim3 grid(c.T, pairs);
    if (dtype == MSR_BF16)
        hipLaunchKernelGGL(generic_output_kernel<uint16_t>, grid, dim3(OUT_THREADS), 0, st, c,
                           chunk, Qr, Kr, static_cast<const uint16_t *>(V),
                           static_cast<uint16_t *>(O), states, pair_stride, chunk_stride);
    else
        hipLaunchKernelGGL(generic_output_kernel<float>, grid, dim3(OUT_THREADS), 0, st, c,
                           chunk, Qr, Kr, static_cast<const float *>(V), static_cast<float *>(O),
                           states, pair_stride, chunk_stride);
    return hipGetLastError();
}

hipError_t launch_copy_state(const MsrConst &c, const float *s_in, float *s_out, hipStream_t st) {
    const size_t n = static_cast<size_t>(c.B) * c.H * c.dk * c.dv;
    if (n == 0 || !s_out) return hipSuccess;
    hipLaunchKernelGGL(copy_state_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, n, s_in,
                       s_out);
    return hipGetLastError();
}
