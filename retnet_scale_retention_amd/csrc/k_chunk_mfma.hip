// k_chunk_mfma.hip -- bf16 matrix-core (MFMA) path of the chunkwise form.
//
// Per chunk i of b tokens (jsqmd.com "From RoPE to Retention" s4.3; aiqz.cc
// RetNet tutorial, "chunkwise recurrence"):
//   O_i = GN( (Q~_i K~_i^T (.) D) V_i + (Q~_i S_{i-1}) (.) xi )
//   S_i = gamma^b S_{i-1} + K~_i^T (V_i (.) zeta)
//
// Work decomposition.  One workgroup owns one (batch, head) pair and one
// slice of W = 64 value columns for the WHOLE sequence; its fp32 state slice
// S[dk][W] lives in MFMA accumulators for the entire run, split over the
// waves by rows of d_k.  Per chunk the workgroup
//   1. stages the chunk's rotated K~ [b][dk] and its V slice [b][W] in LDS
//      (bf16), the rotation read from a per-call cos/sin table;
//   2. state update: S = gamma^b S + K~^T (V (.) zeta s) -- both operands are
//      token-contiguous reads of the row-major LDS tiles, done with the gfx950
//      LDS transpose read (ds_read_b64_tr_b16);
//   3. for its 16 query rows each wave keeps Q~ in registers and computes
//        O^T  = (S_old^T Q~^T) (.) xi                 (S_old^T bf16 in LDS)
//        P^T  = mask(K~ Q~^T) -- decay and scale applied in registers
//        O^T += V^T P^T      -- P^T stays in registers: two 16x16 result
//                              tiles form the next MFMA's B operand once the
//                              keys are taken in the order
//                              {4g..4g+3, 16+4g..16+4g+3} for lane group g,
//                              and V^T is read in that same order;
//      then GroupNorm over d_v (in-wave when W == d_v, else the slice writes
//      its row statistics and a small finalize pass normalises);
//   4. writes S_new^T as bf16 to LDS for the next chunk's inter-chunk term.
// Decay factors gamma^d are exp2(d log2 gamma) with d >= 0, tabulated once
// per workgroup in LDS.
#include "msr_device.hpp"
#include "msr_mfma.hpp"

namespace {

using namespace msr;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int W = 64;  // value columns per workgroup slice

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read: 16 lanes each point at 4 consecutive bf16 of row
// (base_row + j/4) -- lane i receives column (i) of the 4 rows addressed by
// the lanes {i/4, 4 + i/4, 8 + i/4, 12 + i/4}.  With lane j addressing
// &tile[r0 + j/4][c0 + 4 (j%4)], lane i gets tile[r0 + e][c0 + i], e = 0..3.
__device__ __forceinline__ s16x4 lds_tr(const __bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4 *)((__attribute__((address_space(3))) char *)(p)));
}

__device__ __forceinline__ bf16x8 cat(s16x4 a, s16x4 b) {
    s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float bf(short s) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(s)) << 16);
}

__device__ __forceinline__ bf16x8 ld_lds8(const __bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// 8 bf16 from global memory at p (16-byte aligned), rotated pairwise with
// the 4 (cos, sin) entries at cs: (x0 c - x1 s, x1 c + x0 s).
__device__ __forceinline__ bf16x8 load_rot8(const uint16_t *p, const float2 *cs, bool rotate) {
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(p);
    bf16x8 out;
    if (rotate) {
        const float4 c01 = *reinterpret_cast<const float4 *>(cs);
        const float4 c23 = *reinterpret_cast<const float4 *>(cs + 2);
        const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
        const float ss[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x0 = __uint_as_float(raw[i] << 16);
            const float x1 = __uint_as_float(raw[i] & 0xffff0000u);
            out[2 * i] = static_cast<__bf16>(x0 * cc[i] - x1 * ss[i]);
            out[2 * i + 1] = static_cast<__bf16>(x1 * cc[i] + x0 * ss[i]);
        }
    } else {
        out = __builtin_bit_cast(bf16x8, raw);
    }
    return out;
}

template <int DK, int BC>
struct Cfg {
    static constexpr int NW = (BC / 16 < 8 ? BC / 16 : 8) < DK / 16 ? (BC / 16 < 8 ? BC / 16 : 8) : DK / 16;
    static constexpr int THREADS = NW * 64;
    static constexpr int QB = 16 * NW;      // query rows per block
    static constexpr int NQB = BC / QB;     // query blocks per chunk
    static constexpr int RS = DK / NW;      // state rows per wave
    static constexpr int RT = RS / 16;      // state row tiles per wave
    static constexpr int CT = W / 16;       // column tiles
    static constexpr int KS = DK / 32;      // k-steps over d_k
    static constexpr int KP = DK + 8;       // padded LDS row (bf16) of K~
    static constexpr int VP = W + 8;        // padded LDS row of V
    static constexpr int SP = DK + 8;       // padded LDS row of S^T
    static constexpr size_t LDS_BYTES =
        (size_t)BC * KP * 2 + (size_t)BC * VP * 2 + (size_t)W * SP * 2 + 3 * BC * 4;
};

struct ChunkArgs {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    const float *s_in;
    float *s_out;
    const float2 *cs;  // [T][dk/2] cos/sin of (pos0 + t) theta_i
    float2 *stats;     // [B*T*H][NS] (mean, M2) of each slice, when NS > 1
    int NS;            // slices per pair (dv / W)
};

template <int DK, int BC>
__global__ __launch_bounds__((Cfg<DK, BC>::THREADS)) void chunk_mfma_kernel(MsrConst c, ChunkArgs a) {
    using C = Cfg<DK, BC>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __bf16 *Ks = reinterpret_cast<__bf16 *>(smem);                   // [BC][KP]
    __bf16 *Vs = Ks + BC * C::KP;                                      // [BC][VP]
    __bf16 *St = Vs + BC * C::VP;                                      // [W][SP]
    float *dec = reinterpret_cast<float *>(St + W * C::SP);            // scale gamma^d
    float *zet = dec + BC;                                             // scale gamma^(BC-1-t)
    float *xi = zet + BC;                                              // gamma^(j+1)

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    // workgroup -> (pair, slice); consecutive ids run on different XCDs, so
    // the slices of one pair are placed on the same XCD (id % 8 equal).
    const int npairs = c.B * c.H;
    int pair, slice;
    {
        const int id = blockIdx.x;
        if (npairs % 8 == 0) {
            const int xcd = id & 7, j = id >> 3;
            pair = (j / a.NS) * 8 + xcd;
            slice = j % a.NS;
        } else {
            pair = id / a.NS;
            slice = id % a.NS;
        }
    }
    const int b = pair / c.H, h = pair % c.H;
    const int col0 = slice * W;
    const float lg = c.log2g[h];
    const bool rotate = !(c.flags & MSR_FLAG_NO_ROTATE);
    const size_t rowQK = (size_t)c.H * DK;  // elements between tokens in Q, K
    const size_t rowV = (size_t)c.H * c.dv;

    for (int t = tid; t < BC; t += C::THREADS) {
        dec[t] = c.scale * exp2f((float)t * lg);
        zet[t] = c.scale * exp2f((float)(BC - 1 - t) * lg);
        xi[t] = exp2f((float)(t + 1) * lg);
    }
    const float gb = exp2f((float)BC * lg);

    // ---- state slice in accumulators: rows w*RS + rt*16 + 4g + r, col ct*16 + l16
    f32x4 S[C::RT][C::CT];
    const size_t sbase = (size_t)pair * DK * c.dv + col0;
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = w * C::RS + rt * 16 + 4 * g + r;
                S[rt][ct][r] = a.s_in ? a.s_in[sbase + (size_t)row * c.dv + ct * 16 + l16] : 0.f;
            }
    auto write_st = [&]() {
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) {
                __bf16 *dst = St + (ct * 16 + l16) * C::SP + w * C::RS + rt * 16 + 4 * g;
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                bf16x4 v4;
#pragma unroll
                for (int r = 0; r < 4; ++r) v4[r] = static_cast<__bf16>(S[rt][ct][r]);
                *reinterpret_cast<bf16x4 *>(dst) = v4;
            }
    };
    write_st();

    const int nchunks = c.T / BC;
    for (int ci = 0; ci < nchunks; ++ci) {
        const int t0 = ci * BC;
        __syncthreads();  // previous chunk finished with Ks, Vs; St written
        // ---- stage K~ (rotated, unscaled) and the V slice
        for (int e = tid; e < BC * (DK / 8); e += C::THREADS) {
            const int t = e / (DK / 8), d0 = (e % (DK / 8)) * 8;
            const uint16_t *src = a.k + ((size_t)b * c.T + t0 + t) * rowQK + (size_t)h * DK + d0;
            const float2 *cs = a.cs + (size_t)(t0 + t) * (DK / 2) + d0 / 2;
            *reinterpret_cast<bf16x8 *>(Ks + t * C::KP + d0) = load_rot8(src, cs, rotate);
        }
        for (int e = tid; e < BC * (W / 8); e += C::THREADS) {
            const int t = e / (W / 8), d0 = (e % (W / 8)) * 8;
            const uint16_t *src = a.v + ((size_t)b * c.T + t0 + t) * rowV + (size_t)h * c.dv + col0 + d0;
            *reinterpret_cast<u32x4 *>(Vs + t * C::VP + d0) = *reinterpret_cast<const u32x4 *>(src);
        }
        __syncthreads();

        // ---- queries of this wave: O^T = S_old^T Q~^T xi + V^T P^T
        for (int qb = 0; qb < C::NQB; ++qb) {
            const int j0 = qb * C::QB + 16 * w;  // first query row (within chunk) of this wave
            const int jq = j0 + l16;             // this lane's query column
            bf16x8 qreg[C::KS];
            {
                const size_t tq = (size_t)t0 + jq;
                const uint16_t *src = a.q + ((size_t)b * c.T + tq) * rowQK + (size_t)h * DK + 8 * g;
                const float2 *cs = a.cs + tq * (DK / 2) + 4 * g;
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = load_rot8(src + 32 * ks, cs + 16 * ks, rotate);
            }
            f32x4 oacc[C::CT];
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks)
                    acc = mfma16(ld_lds8(St + (ct * 16 + l16) * C::SP + 32 * ks + 8 * g), qreg[ks], acc);
                const float x = xi[jq];
                oacc[ct] = acc * x;
            }
            // intra-chunk keys 0 .. j0+15, in steps of 32
            const int nsteps = (j0 + 16 + 31) / 32;
            for (int s = 0; s < nsteps; ++s) {
                f32x4 p[2];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int kt0 = 32 * s + 16 * half;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if (kt0 <= j0 + 15) {
#pragma unroll
                        for (int ks = 0; ks < C::KS; ++ks)
                            acc = mfma16(ld_lds8(Ks + (kt0 + l16) * C::KP + 32 * ks + 8 * g), qreg[ks], acc);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = kt0 + 4 * g + r;
                        acc[r] = (t <= jq) ? acc[r] * dec[jq - t] : 0.f;
                    }
                    p[half] = acc;
                }
                bf16x8 pb;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pb[r] = static_cast<__bf16>(p[0][r]);
                    pb[4 + r] = static_cast<__bf16>(p[1][r]);
                }
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) {
                    const __bf16 *base = Vs + ct * 16 + 4 * (l16 & 3);
                    const s16x4 lo = lds_tr(base + (32 * s + 4 * g + (l16 >> 2)) * C::VP);
                    const s16x4 hi = lds_tr(base + (32 * s + 16 + 4 * g + (l16 >> 2)) * C::VP);
                    oacc[ct] = mfma16(cat(lo, hi), pb, oacc[ct]);
                }
            }
            // ---- GroupNorm over the row (lanes l16, l16+16, +32, +48 share a query)
            const size_t orow = ((size_t)b * c.T + t0 + jq) * c.H + h;
            float sum = 0.f;
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) sum += oacc[ct][0] + oacc[ct][1] + oacc[ct][2] + oacc[ct][3];
            sum += __shfl_xor(sum, 16, 64);
            sum += __shfl_xor(sum, 32, 64);
            const float mean = sum * (1.f / W);
            float m2 = 0.f;
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) m2 += (oacc[ct][r] - mean) * (oacc[ct][r] - mean);
            m2 += __shfl_xor(m2, 16, 64);
            m2 += __shfl_xor(m2, 32, 64);
            const bool gn = !(c.flags & MSR_FLAG_NO_GROUPNORM);
            float mu = 0.f, inv = 1.f;
            if (gn && a.NS == 1) {
                mu = mean;
                inv = 1.f / sqrtf(m2 * (1.f / W) + c.eps);
            } else if (gn && g == 0) {
                a.stats[orow * a.NS + slice] = make_float2(mean, m2);
            }
            uint16_t *dst = a.o + orow * c.dv + col0 + 4 * g;
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                bf16x4 v4;
#pragma unroll
                for (int r = 0; r < 4; ++r) v4[r] = static_cast<__bf16>((oacc[ct][r] - mu) * inv);
                *reinterpret_cast<bf16x4 *>(dst + ct * 16) = v4;
            }
        }

        // ---- state update S = gamma^b S + K~^T (V zeta s), rows of this wave
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) S[rt][ct] = S[rt][ct] * gb;
        for (int s = 0; s < BC / 32; ++s) {
            bf16x8 bv[C::CT];
            const int tb = 32 * s + 8 * g;  // first token of this lane group
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) {
                const __bf16 *base = Vs + ct * 16 + 4 * (l16 & 3);
                const s16x4 lo = lds_tr(base + (tb + (l16 >> 2)) * C::VP);
                const s16x4 hi = lds_tr(base + (tb + 4 + (l16 >> 2)) * C::VP);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bv[ct][e] = static_cast<__bf16>(bf(lo[e]) * zet[tb + e]);
                    bv[ct][4 + e] = static_cast<__bf16>(bf(hi[e]) * zet[tb + 4 + e]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < C::RT; ++rt) {
                const __bf16 *base = Ks + w * C::RS + rt * 16 + 4 * (l16 & 3);
                const s16x4 lo = lds_tr(base + (tb + (l16 >> 2)) * C::KP);
                const s16x4 hi = lds_tr(base + (tb + 4 + (l16 >> 2)) * C::KP);
                const bf16x8 ak = cat(lo, hi);
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) S[rt][ct] = mfma16(ak, bv[ct], S[rt][ct]);
            }
        }
        __syncthreads();  // every wave is done reading St (old state)
        write_st();
    }

    if (a.s_out) {
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = w * C::RS + rt * 16 + 4 * g + r;
                    a.s_out[sbase + (size_t)row * c.dv + ct * 16 + l16] = S[rt][ct][r];
                }
    }
}

// cos/sin table of (pos0 + t) * theta_i, [T][dk/2] float2.
__global__ void angle_table_kernel(MsrConst c, float2 *cs) {
    const int half = c.dk / 2;
    const size_t n = (size_t)c.T * half;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int i = (int)(e % half);
        const int64_t t = (int64_t)(e / half);
        float co, si;
        rot_cos_sin(c.pos0 + t, c.theta[i], co, si);
        cs[e] = make_float2(co, si);
    }
}

// GroupNorm of rows whose slices wrote (mean, M2) statistics: combines the
// NS slice statistics (Chan et al.'s pairwise update) and normalises the
// d_v values of the row in place.  One wave per row.
__global__ void gn_finalize_kernel(MsrConst c, int NS, const float2 *stats, uint16_t *o, size_t rows) {
    const int lane = threadIdx.x & 63;
    const size_t row = blockIdx.x * (size_t)(blockDim.x / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    float n = 0.f, mean = 0.f, m2 = 0.f;
    for (int s = 0; s < NS; ++s) {
        const float2 st = stats[row * NS + s];
        const float nb = (float)W, nn = n + nb;
        const float d = st.x - mean;
        mean += d * (nb / nn);
        m2 += st.y + d * d * (n * nb / nn);
        n = nn;
    }
    const float inv = 1.f / sqrtf(m2 / n + c.eps);
    uint16_t *p = o + row * c.dv;
    for (int j = lane; j < c.dv; j += 64) p[j] = f32_to_bf16((bf16_to_f32(p[j]) - mean) * inv);
}

template <int DK, int BC>
hipError_t launch_chunk(const MsrConst &c, const ChunkArgs &a, hipStream_t st) {
    using C = Cfg<DK, BC>;
    auto kern = chunk_mfma_kernel<DK, BC>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
    if (e != hipSuccess) return e;
    const int grid = c.B * c.H * a.NS;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), C::LDS_BYTES, st, c, a);
    return hipGetLastError();
}

template <int DK>
hipError_t dispatch_bc(const MsrConst &c, const ChunkArgs &a, int chunk, hipStream_t st) {
    switch (chunk) {
    case 64: return launch_chunk<DK, 64>(c, a, st);
    case 128: return launch_chunk<DK, 128>(c, a, st);
    case 256:
        if constexpr (DK <= 128) return launch_chunk<DK, 256>(c, a, st);
        return hipErrorNotSupported;
    default: return hipErrorNotSupported;
    }
}

struct MfmaPlan {
    size_t cs = 0, stats = 0, total = 0;
};

MfmaPlan mfma_plan(const msr_problem *p) {
    MfmaPlan m;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    m.cs = 0;
    m.stats = up((size_t)p->T * (p->dk / 2) * sizeof(float2));
    const int NS = p->dv / W;
    m.total = m.stats + (NS > 1 ? up((size_t)p->B * p->T * p->H * NS * sizeof(float2)) : 0);
    return m;
}

}  // namespace

bool mfma_supported(const msr_problem *p, int form, int chunk) {
    if (form != MSR_FORM_CHUNKWISE || p->dtype != MSR_BF16) return false;
    if (p->dk != 64 && p->dk != 128 && p->dk != 256) return false;
    if (p->dv % W != 0) return false;
    if (chunk != 64 && chunk != 128 && chunk != 256) return false;
    if (p->dk == 256 && chunk == 256) return false;
    if (chunk > p->T || p->T % chunk != 0) return false;
    return true;
}

size_t mfma_workspace_bytes(const msr_problem *p, int form, int chunk) {
    if (!mfma_supported(p, form, chunk)) return 0;
    return mfma_plan(p).total;
}

hipError_t mfma_chunkwise(const MsrConst &c, const msr_problem *p, int chunk, const void *Q,
                          const void *K, const void *V, void *O, const float *s_in, float *s_out,
                          void *ws, hipStream_t st) {
    const MfmaPlan m = mfma_plan(p);
    char *wsb = static_cast<char *>(ws);
    ChunkArgs a;
    a.q = static_cast<const uint16_t *>(Q);
    a.k = static_cast<const uint16_t *>(K);
    a.v = static_cast<const uint16_t *>(V);
    a.o = static_cast<uint16_t *>(O);
    a.s_in = s_in;
    a.s_out = s_out;
    a.cs = reinterpret_cast<float2 *>(wsb + m.cs);
    a.NS = p->dv / W;
    a.stats = a.NS > 1 ? reinterpret_cast<float2 *>(wsb + m.stats) : nullptr;

    const size_t ncs = (size_t)p->T * (p->dk / 2);
    size_t g = (ncs + 255) / 256;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(angle_table_kernel, dim3((unsigned)g), dim3(256), 0, st, c,
                       reinterpret_cast<float2 *>(wsb + m.cs));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (p->dk) {
    case 64: e = dispatch_bc<64>(c, a, chunk, st); break;
    case 128: e = dispatch_bc<128>(c, a, chunk, st); break;
    case 256: e = dispatch_bc<256>(c, a, chunk, st); break;
    default: e = hipErrorNotSupported;
    }
    if (e != hipSuccess) return e;
    if (a.NS > 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM)) {
        const size_t rows = (size_t)p->B * p->T * p->H;
        const size_t blocks = (rows + 3) / 4;
        hipLaunchKernelGGL(gn_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, a.NS,
                           a.stats, a.o, rows);
        e = hipGetLastError();
    }
    return e;
}

hipError_t mfma_parallel(const MsrConst &, const msr_problem *, const void *, const void *,
                         const void *, void *, const float *, float *, void *, hipStream_t) {
    return hipErrorNotSupported;
}
