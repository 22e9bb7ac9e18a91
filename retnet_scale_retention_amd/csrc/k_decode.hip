// k_decode.hip -- recurrent decode steps of multi-scale retention, one or a
// few tokens per pair and call:
//   S <- gamma S + k~^T v ;  o = GN(q~ S)      (per token, in order)
// (jsqmd.com "From RoPE to Retention" s4.2; aiqz.cc RetNet tutorial,
// "recurrent representation": the output reads the updated state).
// Up to MSR_DECODE_MAX_T tokens share one pass over the state: the
// single-token step and short chunkwise calls (multi-token serving steps).
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

// The single-token step, state updated in place (the decode hot path; kept
// separate from the multi-token kernel below, which is ~3% slower at one
// token).
template <typename TIn>
__global__ __launch_bounds__(DEC_THREADS) void decode_step_kernel(MsrConst c, const TIn *__restrict__ q,
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
    if (c.flags & MSR_FLAG_DECAY_ROWNORM) {
        const float f = row_norm_factor(c, row_pos0(c, pair / c.H), c.log2g[h]);
        out.x *= f;
        out.y *= f;
        out.z *= f;
        out.w *= f;
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

// NT tokens per pair (the recurrent form over T <= NT tokens, T = c.T):
//   for t: S <- gamma S + k~_t^T v_t ;  o_t = GN(q~_t S)
// with the state streamed from HBM once: each row of S takes all T updates
// while it is in registers, and each token's partial output sums q~_t[i] S[i]
// over the thread's rows.  Token t of pair (b, h) sits at ((b T + t) H + h)
// in Q, K, V and O.  s_in NULL means a zero state; s_out NULL drops the final
// state (it may equal s_in: each element is read and then written by the
// same thread).
template <typename TIn, int NT>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(MsrConst c, const TIn *__restrict__ q,
                                                             const TIn *__restrict__ k,
                                                             const TIn *__restrict__ v,
                                                             TIn *__restrict__ o, const float *s_in,
                                                             float *s_out) {
    const int pair = blockIdx.x, b = pair / c.H, h = pair % c.H;
    const int tid = threadIdx.x;
    const int T = NT == 1 ? 1 : c.T;  // 1 <= T <= NT (known at compile time for one token)
    __shared__ float qs[NT][MSR_MAX_DK];
    __shared__ float ks[NT][MSR_MAX_DK];
    __shared__ float4 part[DEC_THREADS];
    __shared__ float red[16];

    const int G = c.dv / 4;        // float4 column groups per row (<= 256)
    const int R = DEC_THREADS / G; // row groups
    const int rg = tid / G, cg = tid - rg * G;
    const bool active = rg < R;
    const size_t soff = static_cast<size_t>(pair) * c.dk * c.dv;
    const f32x4 *Si = s_in ? reinterpret_cast<const f32x4 *>(s_in + soff) : nullptr;
    f32x4 *So = s_out ? reinterpret_cast<f32x4 *>(s_out + soff) : nullptr;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // a batch of DEC_U state rows (the null-state test stays outside the
    // unrolled loads, so that all of them are in flight together)
    f32x4 s[DEC_U];
    auto load_batch = [&](int i0) {
        if (Si) {
#pragma unroll
            for (int u = 0; u < DEC_U; ++u) {
                const int i = i0 + u * R;
                if (i < c.dk) s[u] = __builtin_nontemporal_load(&Si[static_cast<size_t>(i) * G + cg]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < DEC_U; ++u) s[u] = zero4;
        }
    };
    // the first batch is in flight during the prologue
    if (active) load_batch(rg);

    // rotated q~, and k~ times the scale, of every token, into LDS
    const int64_t p0 = row_pos0(c, b);
    for (int e = tid; e < T * (c.dk / 2); e += DEC_THREADS) {
        const int t = e / (c.dk / 2), i = e - t * (c.dk / 2);
        const size_t base = ((static_cast<size_t>(b) * T + t) * c.H + h) * c.dk;
        const float q0 = load(q, base + 2 * i), q1 = load(q, base + 2 * i + 1);
        const float k0 = load(k, base + 2 * i), k1 = load(k, base + 2 * i + 1);
        float cs = 1.f, sn = 0.f;
        if (!(c.flags & MSR_FLAG_NO_ROTATE)) rot_cos_sin(p0 + t, c.theta[i], cs, sn);
        qs[t][2 * i] = q0 * cs - q1 * sn;
        qs[t][2 * i + 1] = q1 * cs + q0 * sn;
        ks[t][2 * i] = (k0 * cs - k1 * sn) * c.scale;
        ks[t][2 * i + 1] = (k1 * cs + k0 * sn) * c.scale;
    }
    __syncthreads();

    const float g = c.gamma[h];
    f32x4 acc[NT], vv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        acc[t] = zero4;
        vv[t] = zero4;
        if (active && t < T) {
            const size_t vb = ((static_cast<size_t>(b) * T + t) * c.H + h) * c.dv + 4 * cg;
            vv[t] = f32x4{load(v, vb), load(v, vb + 1), load(v, vb + 2), load(v, vb + 3)};
        }
    }
    if (active) {
        for (int i0 = rg; i0 < c.dk; i0 += R * DEC_U) {
            if (i0 != rg) load_batch(i0);  // the first batch is already loaded
#pragma unroll
            for (int u = 0; u < DEC_U; ++u) {
                const int i = i0 + u * R;
                if (i < c.dk) {
                    f32x4 x = s[u];
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        if (t < T) {
                            const float ki = ks[t][i], qi = qs[t][i];
                            x = g * x + ki * vv[t];
                            acc[t] += qi * x;
                        }
                    }
                    s[u] = x;
                }
            }
            if (So) {
#pragma unroll
                for (int u = 0; u < DEC_U; ++u) {
                    const int i = i0 + u * R;
                    if (i < c.dk) __builtin_nontemporal_store(s[u], &So[static_cast<size_t>(i) * G + cg]);
                }
            }
        }
    }

    // per token: the row groups' partial sums meet in LDS, then GroupNorm
    for (int t = 0; t < T; ++t) {
        f32x4 a = zero4;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            if (tt == t) a = acc[tt];
        part[tid] = float4{a.x, a.y, a.z, a.w};
        __syncthreads();
        // thread cg < G sums the R partials of its column group
        float4 out = make_float4(0.f, 0.f, 0.f, 0.f);
        const bool owner = tid < G;
        if (owner) {
            for (int r = 0; r < R; ++r) {
                const float4 pv = part[r * G + tid];
                out.x += pv.x;
                out.y += pv.y;
                out.z += pv.z;
                out.w += pv.w;
            }
        }
        if (c.flags & MSR_FLAG_DECAY_ROWNORM) {
            const float f = row_norm_factor(c, p0 + t, c.log2g[h]);
            out.x *= f;
            out.y *= f;
            out.z *= f;
            out.w *= f;
        }
        if (!(c.flags & MSR_FLAG_NO_GROUPNORM)) {
            const float sm = owner ? (out.x + out.y + out.z + out.w) : 0.f;
            const float mean = block_sum(sm, red) / c.dv;
            float q2 = 0.f;
            if (owner) {
                const float d0 = out.x - mean, d1 = out.y - mean, d2 = out.z - mean, d3 = out.w - mean;
                q2 = d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
            }
            const float var = block_sum(q2, red) / c.dv;
            const float inv = 1.f / sqrtf(var + c.eps);
            out.x = (out.x - mean) * inv;
            out.y = (out.y - mean) * inv;
            out.z = (out.z - mean) * inv;
            out.w = (out.w - mean) * inv;
        }
        if (owner) {
            const size_t ob = ((static_cast<size_t>(b) * T + t) * c.H + h) * c.dv + 4 * tid;
            store(o, ob, out.x);
            store(o, ob + 1, out.y);
            store(o, ob + 2, out.z);
            store(o, ob + 3, out.w);
        }
        __syncthreads();  // part is rewritten for the next token
    }
}

template <typename TIn, int NT>
void launch_nt(const MsrConst &c, const void *q, const void *k, const void *v, void *o, const float *s_in,
               float *s_out, hipStream_t st) {
    auto kern = decode_kernel<TIn, NT>;
    launch_main(kern, dim3(c.B * c.H), dim3(DEC_THREADS), st, c, static_cast<const TIn *>(q),
                static_cast<const TIn *>(k), static_cast<const TIn *>(v), static_cast<TIn *>(o), s_in, s_out);
}

template <typename TIn>
void launch_tokens(const MsrConst &c, const void *q, const void *k, const void *v, void *o, const float *s_in,
                   float *s_out, hipStream_t st) {
    if (c.T <= 1)
        launch_nt<TIn, 1>(c, q, k, v, o, s_in, s_out, st);
    else if (c.T <= 4)
        launch_nt<TIn, 4>(c, q, k, v, o, s_in, s_out, st);
    else
        launch_nt<TIn, MSR_DECODE_MAX_T>(c, q, k, v, o, s_in, s_out, st);
}

}  // namespace

hipError_t launch_decode(const MsrConst &c, int dtype, const void *q, const void *k, const void *v, void *o,
                         const float *s_in, float *s_out, hipStream_t st) {
    if (c.B * c.H == 0 || c.T == 0) return hipSuccess;
    if (c.T > MSR_DECODE_MAX_T) return hipErrorInvalidValue;
    if (c.T == 1 && s_in && s_in == s_out) {  // one step in place
        const int pairs = c.B * c.H;
        if (dtype == MSR_BF16)
            launch_main(decode_step_kernel<uint16_t>, dim3(pairs), dim3(DEC_THREADS), st, c,
                        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                        static_cast<const uint16_t *>(v), static_cast<uint16_t *>(o), s_out);
        else
            launch_main(decode_step_kernel<float>, dim3(pairs), dim3(DEC_THREADS), st, c,
                        static_cast<const float *>(q), static_cast<const float *>(k),
                        static_cast<const float *>(v), static_cast<float *>(o), s_out);
        return hipGetLastError();
    }
    if (dtype == MSR_BF16)
        launch_tokens<uint16_t>(c, q, k, v, o, s_in, s_out, st);
    else
        launch_tokens<float>(c, q, k, v, o, s_in, s_out, st);
    return hipGetLastError();
}
