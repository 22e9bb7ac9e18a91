// k_decode.hip -- one recurrent decode step of multi-scale retention:
//   S <- gamma S + k~^T v ;  o = GN(q~ S)
// (jsqmd.com "From RoPE to Retention" s4.2; aiqz.cc RetNet tutorial,
// "recurrent representation": the output reads the updated state).
//
// The step is bound by HBM: every call reads and writes the whole fp32
// state (B*H*dk*dv*8 bytes) and does 4 flops per state element.  One
// workgroup per (batch, head) pair streams that pair's state once, in place,
// with 16-byte non-temporal accesses: thread (rg, cg) owns columns
// 4cg..4cg+3 and rows rg, rg+R, ... (R = 512 / (dv/4) row groups), so every
// wave reads whole contiguous rows.  Rows are processed in batches of U = 16
// so that 16 loads are in flight per thread before the first dependent
// store; the first batch is issued before the rotation prologue, whose
// latency it hides.  q~ and k~ (rotated, K scaled) are built once per
// workgroup in LDS; the partial q~ S sums of the row groups meet in LDS,
// then GroupNorm runs over the d_v outputs.
#include "msr_device.hpp"

namespace {

using namespace msr;

constexpr int DEC_THREADS = 512;
constexpr int DEC_U = 16;
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename TIn>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(MsrConst c, const TIn *__restrict__ q,
                                                             const TIn *__restrict__ k,
                                                             const TIn *__restrict__ v,
                                                             TIn *__restrict__ o,
                                                             float *__restrict__ state) {
    const int pair = blockIdx.x, h = pair % c.H;
    const int tid = threadIdx.x;
    __shared__ float qs[MSR_MAX_DK];
    __shared__ float ks[MSR_MAX_DK];
    __shared__ float4 part[DEC_THREADS];
    __shared__ float red[16];

    const int G = c.dv / 4;        // float4 column groups per row (<= 256)
    const int R = DEC_THREADS / G; // row groups
    const int rg = tid / G, cg = tid - rg * G;
    const bool active = rg < R;
    f32x4 *S4 = reinterpret_cast<f32x4 *>(state + static_cast<size_t>(pair) * c.dk * c.dv);
    // first batch of state rows, in flight during the prologue
    f32x4 s[DEC_U];
    if (active) {
#pragma unroll
        for (int u = 0; u < DEC_U; ++u) {
            const int i = rg + u * R;
            if (i < c.dk) s[u] = __builtin_nontemporal_load(&S4[static_cast<size_t>(i) * G + cg]);
        }
    }

    const size_t qk_base = static_cast<size_t>(pair) * c.dk;
    for (int i = tid; i < c.dk / 2; i += DEC_THREADS) {
        const float q0 = load(q, qk_base + 2 * i), q1 = load(q, qk_base + 2 * i + 1);
        const float k0 = load(k, qk_base + 2 * i), k1 = load(k, qk_base + 2 * i + 1);
        float cs = 1.f, sn = 0.f;
        if (!(c.flags & MSR_FLAG_NO_ROTATE)) rot_cos_sin(row_pos0(c, pair / c.H), c.theta[i], cs, sn);
        qs[2 * i] = q0 * cs - q1 * sn;
        qs[2 * i + 1] = q1 * cs + q0 * sn;
        ks[2 * i] = (k0 * cs - k1 * sn) * c.scale;
        ks[2 * i + 1] = (k1 * cs + k0 * sn) * c.scale;
    }
    __syncthreads();

    const float g = c.gamma[h];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (active) {
        const size_t vb = static_cast<size_t>(pair) * c.dv + 4 * cg;
        const float4 vv = make_float4(load(v, vb), load(v, vb + 1), load(v, vb + 2), load(v, vb + 3));
        for (int i0 = rg; i0 < c.dk; i0 += R * DEC_U) {
            if (i0 != rg) {  // the first batch is already loaded
#pragma unroll
                for (int u = 0; u < DEC_U; ++u) {
                    const int i = i0 + u * R;
                    if (i < c.dk) s[u] = __builtin_nontemporal_load(&S4[static_cast<size_t>(i) * G + cg]);
                }
            }
#pragma unroll
            for (int u = 0; u < DEC_U; ++u) {
                const int i = i0 + u * R;
                if (i < c.dk) {
                    const float ki = ks[i], qi = qs[i];
                    f32x4 x = s[u];
                    x.x = g * x.x + ki * vv.x;
                    x.y = g * x.y + ki * vv.y;
                    x.z = g * x.z + ki * vv.z;
                    x.w = g * x.w + ki * vv.w;
                    __builtin_nontemporal_store(x, &S4[static_cast<size_t>(i) * G + cg]);
                    acc.x += qi * x.x;
                    acc.y += qi * x.y;
                    acc.z += qi * x.z;
                    acc.w += qi * x.w;
                }
            }
        }
    }
    part[tid] = acc;
    __syncthreads();

    // thread cg < G sums the R partials of its column group
    float4 out = make_float4(0.f, 0.f, 0.f, 0.f);
    const bool owner = tid < G;
    if (owner) {
        for (int r = 0; r < R; ++r) {
            const float4 p = part[r * G + tid];
            out.x += p.x;
            out.y += p.y;
            out.z += p.z;
            out.w += p.w;
        }
    }
    if (!(c.flags & MSR_FLAG_NO_GROUPNORM)) {
        const float s = owner ? (out.x + out.y + out.z + out.w) : 0.f;
        const float mean = block_sum(s, red) / c.dv;
        float q2 = 0.f;
        if (owner) {
            const float a = out.x - mean, b2 = out.y - mean, cc = out.z - mean, d = out.w - mean;
            q2 = a * a + b2 * b2 + cc * cc + d * d;
        }
        const float var = block_sum(q2, red) / c.dv;
        const float inv = 1.f / sqrtf(var + c.eps);
        out.x = (out.x - mean) * inv;
        out.y = (out.y - mean) * inv;
        out.z = (out.z - mean) * inv;
        out.w = (out.w - mean) * inv;
    }
    if (owner) {
        const size_t ob = static_cast<size_t>(pair) * c.dv + 4 * tid;
        store(o, ob, out.x);
        store(o, ob + 1, out.y);
        store(o, ob + 2, out.z);
        store(o, ob + 3, out.w);
    }
}

}  // namespace

hipError_t launch_decode(const MsrConst &c, int dtype, const void *q, const void *k,
                         const void *v, void *o, float *state, hipStream_t st) {
    const int pairs = c.B * c.H;
    if (pairs == 0) return hipSuccess;
    if (dtype == MSR_BF16)
        hipLaunchKernelGGL(decode_kernel<uint16_t>, dim3(pairs), dim3(DEC_THREADS), 0, st, c,
                           static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                           static_cast<const uint16_t *>(v), static_cast<uint16_t *>(o), state);
    else
        hipLaunchKernelGGL(decode_kernel<float>, dim3(pairs), dim3(DEC_THREADS), 0, st, c,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), static_cast<float *>(o), state);
    return hipGetLastError();
}
