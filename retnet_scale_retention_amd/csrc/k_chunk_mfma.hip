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

template <int DK, int BC>
struct Cfg {
    static constexpr int NKT = BC / 16;                  // 16-token tiles per chunk
    static constexpr int NW = NKT < 8 ? NKT : 8;         // waves
    static constexpr int NQT = NKT / NW;                 // query tiles per wave (1 or 2)
    static constexpr int THREADS = NW * 64;
    static constexpr int CT = W / 16;          // state / output column tiles
    static constexpr int NT = (DK / 16) * CT;  // state tiles per workgroup
    static constexpr int TPW = NT / NW;        // state tiles per wave
    static constexpr int CPW = TPW < CT ? TPW : CT;  // ... of which column tiles
    static constexpr int RPW = TPW / CPW;            // ... and row tiles
    static constexpr int CG = CT / CPW;              // column groups of waves
    static constexpr int KS = DK / 32;      // k-steps over d_k
    static constexpr int XP = DK + 8;       // padded LDS row (bf16) of Q~ / K~
    static constexpr int VP = W + 8;        // padded LDS row of V
    static constexpr int SP = DK + 8;       // padded LDS row of S^T
    static constexpr int PAIRS8 = DK / 8;   // 8-element pieces per Q/K row
    static constexpr int ITER = BC * PAIRS8 / THREADS;  // Q/K pieces per thread per chunk
    static constexpr int TSTRIDE = THREADS / PAIRS8;    // token stride between them
    static constexpr int VITER = BC * (W / 8) / THREADS;
    static constexpr size_t LDS_BYTES = (size_t)BC * XP * 2 + 2 * (size_t)BC * VP * 2 +
                                        (size_t)W * SP * 2 + 2 * BC * 4;
    static_assert(NKT % NW == 0 && NQT <= 2, "query tiles split over waves");
    static_assert(NT % NW == 0 && TPW >= 1, "state tiles must split evenly over waves");
    static_assert(BC * PAIRS8 % THREADS == 0 && THREADS % PAIRS8 == 0, "staging split");
    static_assert(BC * (W / 8) % THREADS == 0, "V staging split");
    static_assert(LDS_BYTES <= 163840, "LDS budget");
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Rotate 4 channel pairs (8 bf16 packed in u) by the angles with cos/sin
// (cc[i], ss[i]): (x0 c - x1 s, x1 c + x0 s) in fp32, rounded to bf16.
__device__ __forceinline__ u32x4 rot4(u32x4 u, const float *cc, const float *ss) {
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x0 = __uint_as_float(u[i] << 16);
        const float x1 = __uint_as_float(u[i] & 0xffff0000u);
        const bf16x2 y = {static_cast<__bf16>(x0 * cc[i] - x1 * ss[i]),
                          static_cast<__bf16>(x1 * cc[i] + x0 * ss[i])};
        out[i] = __builtin_bit_cast(uint32_t, y);
    }
    return out;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2 y = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, y);
}

template <int DK, int BC>
__global__ __launch_bounds__((Cfg<DK, BC>::THREADS)) void chunk_mfma_kernel(MsrConst c, ChunkArgs a) {
    using C = Cfg<DK, BC>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __bf16 *Xs = reinterpret_cast<__bf16 *>(smem);                   // [BC][XP]  Q~, then K~
    __bf16 *Vs = Xs + BC * C::XP;                                      // [BC][VP]  V
    __bf16 *Vz = Vs + BC * C::VP;                                      // [BC][VP]  V zeta s
    __bf16 *St = Vz + BC * C::VP;                                      // [W][SP]   S_old^T
    float *dec = reinterpret_cast<float *>(St + W * C::SP);            // s gamma^d
    float *xi = dec + BC;                                              // gamma^(j+1)

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    // workgroup -> (pair, slice): the slices of one pair get ids equal mod 8,
    // i.e. run on the same XCD and share its L2 for the Q and K chunks.
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
        xi[t] = exp2f((float)(t + 1) * lg);
    }
    const float gb = exp2f((float)BC * lg);

    // ---- staging assignment: this thread owns channel pairs p0..p0+3 of
    // tokens tf, tf + TSTRIDE, ... of every chunk (same pairs for Q and K).
    const int tf = tid / C::PAIRS8;
    const int d0 = (tid % C::PAIRS8) * 8;
    float stc[4], sts[4];  // cos/sin of TSTRIDE * theta for the 4 pairs
#pragma unroll
    for (int i = 0; i < 4; ++i) rot_cos_sin(C::TSTRIDE, c.theta[d0 / 2 + i], stc[i], sts[i]);
    const int vt0 = tid / (W / 8), vd0 = (tid % (W / 8)) * 8;
    constexpr int VSTRIDE = C::THREADS / (W / 8);

    // zeta s for this thread's V tokens (same in every chunk)
    float zv[C::VITER];
#pragma unroll
    for (int it = 0; it < C::VITER; ++it)
        zv[it] = c.scale * exp2f((float)(BC - 1 - (vt0 + it * VSTRIDE)) * lg);

    u32x4 rq[C::ITER], rk[C::ITER], rv[C::VITER];
    float2 cs0[4];
    // raw Q (issued late, after the MFMA work of a chunk) and raw K, V and
    // the first cos/sin (issued right after staging) of the next chunk
    auto prefetch_q = [&](int t0) {
        const size_t tok = (size_t)b * c.T + t0 + tf;
#pragma unroll
        for (int it = 0; it < C::ITER; ++it)
            rq[it] = *reinterpret_cast<const u32x4 *>(a.q + (tok + (size_t)it * C::TSTRIDE) * rowQK +
                                                      (size_t)h * DK + d0);
    };
    auto prefetch_kv = [&](int t0) {
        const size_t tok = (size_t)b * c.T + t0 + tf;
#pragma unroll
        for (int it = 0; it < C::ITER; ++it)
            rk[it] = *reinterpret_cast<const u32x4 *>(a.k + (tok + (size_t)it * C::TSTRIDE) * rowQK +
                                                      (size_t)h * DK + d0);
        const size_t tokv = (size_t)b * c.T + t0 + vt0;
#pragma unroll
        for (int it = 0; it < C::VITER; ++it)
            rv[it] = *reinterpret_cast<const u32x4 *>(
                a.v + (tokv + (size_t)it * VSTRIDE) * rowV + (size_t)h * c.dv + col0 + vd0);
        const float4 *cp = reinterpret_cast<const float4 *>(a.cs + (size_t)(t0 + tf) * (DK / 2) + d0 / 2);
        const float4 c01 = cp[0], c23 = cp[1];
        cs0[0] = make_float2(c01.x, c01.y);
        cs0[1] = make_float2(c01.z, c01.w);
        cs0[2] = make_float2(c23.x, c23.y);
        cs0[3] = make_float2(c23.z, c23.w);
    };

    // ---- state tiles of this wave: rows (rg*RPW + rt)*16 + 4g + r, cols (cg*CPW + ct)*16 + l16
    const int cgw = w % C::CG, rgw = w / C::CG;
    f32x4 S[C::RPW][C::CPW];
    const size_t sbase = (size_t)pair * DK * c.dv + col0;
#pragma unroll
    for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = (rgw * C::RPW + rt) * 16 + 4 * g + r;
                const int col = (cgw * C::CPW + ct) * 16 + l16;
                S[rt][ct][r] = a.s_in ? a.s_in[sbase + (size_t)row * c.dv + col] : 0.f;
            }
    auto write_st = [&]() {
#pragma unroll
        for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct) {
                const int row = (rgw * C::RPW + rt) * 16 + 4 * g;
                const int col = (cgw * C::CPW + ct) * 16 + l16;
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                bf16x4 v4;
#pragma unroll
                for (int r = 0; r < 4; ++r) v4[r] = static_cast<__bf16>(S[rt][ct][r]);
                *reinterpret_cast<bf16x4 *>(St + col * C::SP + row) = v4;
            }
    };

    prefetch_q(0);
    prefetch_kv(0);
    write_st();

    const int nchunks = c.T / BC;
    // query tiles of this wave: w and, when there are two, NKT-1-w (balances
    // the causal work between waves)
    int qtile[C::NQT];
    qtile[0] = w;
    if (C::NQT == 2) qtile[C::NQT - 1] = C::NKT - 1 - w;
    for (int ci = 0; ci < nchunks; ++ci) {
        const int t0 = ci * BC;
        // ---- rotate Q and K pieces (cos/sin advanced by TSTRIDE per piece)
        if (rotate) {
            float cc[4], ss[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cc[i] = cs0[i].x;
                ss[i] = cs0[i].y;
            }
#pragma unroll
            for (int it = 0; it < C::ITER; ++it) {
                rq[it] = rot4(rq[it], cc, ss);
                rk[it] = rot4(rk[it], cc, ss);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float nc = cc[i] * stc[i] - ss[i] * sts[i];
                    const float ns = ss[i] * stc[i] + cc[i] * sts[i];
                    cc[i] = nc;
                    ss[i] = ns;
                }
            }
        }
#pragma unroll
        for (int it = 0; it < C::ITER; ++it)
            *reinterpret_cast<u32x4 *>(Xs + (tf + it * C::TSTRIDE) * C::XP + d0) = rq[it];
        __syncthreads();  // Q~ staged; St holds S_old
        bf16x8 qreg[C::NQT][C::KS];
#pragma unroll
        for (int u = 0; u < C::NQT; ++u)
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                qreg[u][ks] = ld_lds8(Xs + (16 * qtile[u] + l16) * C::XP + 32 * ks + 8 * g);
        __syncthreads();  // every wave has its Q~ rows
#pragma unroll
        for (int it = 0; it < C::ITER; ++it)
            *reinterpret_cast<u32x4 *>(Xs + (tf + it * C::TSTRIDE) * C::XP + d0) = rk[it];
#pragma unroll
        for (int it = 0; it < C::VITER; ++it) {
            const int t = vt0 + it * VSTRIDE;
            *reinterpret_cast<u32x4 *>(Vs + t * C::VP + vd0) = rv[it];
            u32x4 z;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                z[i] = pack_bf16x2(__uint_as_float(rv[it][i] << 16) * zv[it],
                                   __uint_as_float(rv[it][i] & 0xffff0000u) * zv[it]);
            *reinterpret_cast<u32x4 *>(Vz + t * C::VP + vd0) = z;
        }
        if (ci + 1 < nchunks) prefetch_kv(t0 + BC);  // next chunk's loads fly during the compute
        __syncthreads();  // K~, V, V zeta staged

        // ---- state update S = gamma^b S + K~^T (V zeta s) on this wave's tiles
#pragma unroll
        for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = S[rt][ct] * gb;
#pragma unroll 2
        for (int s = 0; s < BC / 32; ++s) {
            const int tb = 32 * s + 8 * g;  // first token of this lane group
            bf16x8 bv[C::CPW];
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct) {
                const __bf16 *base = Vz + (cgw * C::CPW + ct) * 16 + 4 * (l16 & 3);
                bv[ct] = cat(lds_tr(base + (tb + (l16 >> 2)) * C::VP),
                             lds_tr(base + (tb + 4 + (l16 >> 2)) * C::VP));
            }
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt) {
                const __bf16 *base = Xs + (rgw * C::RPW + rt) * 16 + 4 * (l16 & 3);
                const bf16x8 ak = cat(lds_tr(base + (tb + (l16 >> 2)) * C::XP),
                                      lds_tr(base + (tb + 4 + (l16 >> 2)) * C::XP));
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = mfma16(ak, bv[ct], S[rt][ct]);
            }
        }

#pragma unroll
        for (int u = 0; u < C::NQT; ++u) {
            const int qt = qtile[u];
            const int jq = 16 * qt + l16;  // this lane's query row within the chunk
            // ---- O^T = (S_old^T Q~^T) xi   (four independent accumulators)
            f32x4 oacc[C::CT];
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct)
                    oacc[ct] = mfma16(ld_lds8(St + (ct * 16 + l16) * C::SP + 32 * ks + 8 * g), qreg[u][ks],
                                      oacc[ct]);
            {
                const float x = xi[jq];
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = oacc[ct] * x;
            }
            // ---- intra-chunk part, keys 0 .. 16qt+15, four key tiles at a time:
            // P^T tiles (decay, scale and causal mask in registers) packed as
            // B operands, then O^T += V^T P^T
#pragma unroll 1
            for (int kq = 0; kq < C::NKT; kq += 4) {
                if (kq <= qt) {
                    f32x4 acc[4];
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4) acc[v4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
                        for (int v4 = 0; v4 < 4; ++v4)
                            if (kq + v4 <= qt)
                                acc[v4] = mfma16(ld_lds8(Xs + (16 * (kq + v4) + l16) * C::XP + 32 * ks + 8 * g),
                                                 qreg[u][ks], acc[v4]);
                    bf16x8 pb[2];
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = 16 * (kq + v4) + 4 * g + r;
                            const float x = (t <= jq) ? acc[v4][r] * dec[jq - t] : 0.f;
                            pb[v4 / 2][4 * (v4 & 1) + r] = static_cast<__bf16>(x);
                        }
#pragma unroll
                    for (int hs = 0; hs < 2; ++hs) {
                        const int s = kq / 2 + hs;
                        if (2 * s <= qt) {
#pragma unroll
                            for (int ct = 0; ct < C::CT; ++ct) {
                                const __bf16 *base = Vs + ct * 16 + 4 * (l16 & 3);
                                const s16x4 lo = lds_tr(base + (32 * s + 4 * g + (l16 >> 2)) * C::VP);
                                const s16x4 hi = lds_tr(base + (32 * s + 16 + 4 * g + (l16 >> 2)) * C::VP);
                                oacc[ct] = mfma16(cat(lo, hi), pb[hs], oacc[ct]);
                            }
                        }
                    }
                }
            }
            if (u == C::NQT - 1 && ci + 1 < nchunks) prefetch_q(t0 + BC);
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
        __syncthreads();  // every wave is done with Xs, Vs, Vz and St
        write_st();
    }

    if (a.s_out) {
#pragma unroll
        for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = (rgw * C::RPW + rt) * 16 + 4 * g + r;
                    const int col = (cgw * C::CPW + ct) * 16 + l16;
                    a.s_out[sbase + (size_t)row * c.dv + col] = S[rt][ct][r];
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
// NS slice statistics (Chan, Golub and LeVeque's pairwise update) once per
// row, then normalises the row's d_v values in place, 8 values (16 bytes)
// per thread.  A block of 256 threads covers RB = 256 / (d_v / 8) rows.
__global__ __launch_bounds__(256) void gn_finalize_kernel(MsrConst c, int NS, const float2 *stats,
                                                          uint16_t *o, size_t rows) {
    __shared__ float2 mi[256];
    const int tpr = c.dv / 8;          // threads per row
    const int RB = 256 / tpr;          // rows per block
    const size_t row0 = blockIdx.x * (size_t)RB;
    if (threadIdx.x < RB && row0 + threadIdx.x < rows) {
        const size_t row = row0 + threadIdx.x;
        float n = 0.f, mean = 0.f, m2 = 0.f;
        for (int s = 0; s < NS; ++s) {
            const float2 st = stats[row * NS + s];
            const float nb = (float)W, nn = n + nb;
            const float d = st.x - mean;
            mean += d * (nb / nn);
            m2 += st.y + d * d * (n * nb / nn);
            n = nn;
        }
        mi[threadIdx.x] = make_float2(mean, 1.f / sqrtf(m2 / n + c.eps));
    }
    __syncthreads();
    const int r = threadIdx.x / tpr, j = threadIdx.x % tpr;
    if (r >= RB || row0 + r >= rows) return;
    const float mean = mi[r].x, inv = mi[r].y;
    u32x4 *p = reinterpret_cast<u32x4 *>(o + (row0 + r) * c.dv) + j;
    u32x4 u = *p;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        u[i] = pack_bf16x2((__uint_as_float(u[i] << 16) - mean) * inv,
                           (__uint_as_float(u[i] & 0xffff0000u) - mean) * inv);
    *p = u;
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
        const int RB = 256 / (p->dv / 8);
        const size_t blocks = (rows + RB - 1) / RB;
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
