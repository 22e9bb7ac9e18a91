// k_chunk_mfma.hip -- bf16 matrix-core (MFMA) path of the chunkwise form.
//
// Per chunk i of b tokens (jsqmd.com "From RoPE to Retention" s4.3; aiqz.cc
// RetNet tutorial, "chunkwise recurrence"):
//   O_i = GN( (Q~_i K~_i^T (.) D) V_i + (Q~_i S_{i-1}) (.) xi )
//   S_i = gamma^b S_{i-1} + K~_i^T (V_i (.) zeta)
//
// Kernels, in launch order:
//   angle_table_kernel  cos/sin of (pos0 + t) theta_i for every position
//   rotate_qk_kernel    Q~, K~ = theta_shift(Q), theta_shift(K) as bf16, once
//                       per token and head (bandwidth bound)
//   chunk_mfma_kernel   the chunk recurrence, below
//   gn_finalize_kernel  GroupNorm when d_v spans several slices
//
// Work decomposition of chunk_mfma_kernel.  One workgroup owns one (batch,
// head) pair and one slice of W = 64 value columns for the WHOLE sequence;
// its fp32 state slice S[dk][W] lives in MFMA accumulators for the entire
// run, split over the waves in 16x16 tiles.  Per chunk the workgroup
//   1. stages the chunk's K~ [b][dk], its V slice [b][W] and V (.) zeta s in
//      LDS (bf16); each wave holds the Q~ rows of its query tiles in registers
//      (loaded straight from memory in MFMA operand layout); all of it was
//      prefetched into registers during the previous chunk;
//   2. state update: S = gamma^b S + K~^T (V (.) zeta s) -- both operands are
//      token-contiguous reads of the row-major LDS tiles, done with the gfx950
//      LDS transpose read (ds_read_b64_tr_b16);
//   3. per query tile of 16 rows:
//        O^T  = (S_old^T Q~^T) (.) xi                 (S_old^T bf16 in LDS)
//        P^T  = mask(K~ Q~^T) -- decay and scale applied in registers
//        O^T += V^T P^T      -- P^T stays in registers: two 16x16 result
//                              tiles form the next MFMA's B operand once the
//                              keys are taken in the order
//                              {4g..4g+3, 16+4g..16+4g+3} for lane group g,
//                              and V^T is read in that same order;
//      then GroupNorm over d_v (in-wave when W == d_v, else the slice writes
//      its row statistics and the finalize pass normalises);
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
    static constexpr int KB = 32;                        // keys per LDS block (one k-step)
    static constexpr int NB = BC / KB;                   // key blocks per chunk
    static constexpr int NKT = BC / 16;                  // 16-token tiles per chunk
    // waves and query tiles per wave: two tiles per wave (fragment reuse)
    // except for the smallest chunk
    static constexpr int NQT = NKT >= 8 ? 2 : 1;
    static constexpr int NW = NKT / NQT;
    static constexpr int THREADS = NW * 64;
    static constexpr int CT = W / 16;          // state / output column tiles
    static constexpr int NT = (DK / 16) * CT;  // state tiles per workgroup
    static constexpr int TPW = NT / NW;        // state tiles per wave
    static constexpr int CPW = TPW < CT ? TPW : CT;  // ... of which column tiles
    static constexpr int RPW = TPW / CPW;            // ... and row tiles
    static constexpr int CG = CT / CPW;              // column groups of waves
    static constexpr int KS = DK / 32;      // k-steps over d_k
    static constexpr int KROW = DK * 2;     // bytes per K~ / Q~ row in LDS (swizzled)
    static constexpr int KBLK = KB * KROW;  // bytes per K~ block
    static constexpr int VROW = W * 2;      // bytes per V row
    static constexpr int VBLK = KB * VROW;  // bytes per V block
    static constexpr bool QLDS = BC * DK <= 32768;   // next chunk's Q~ staged in LDS
    static constexpr int QBLK = QLDS ? BC * KROW : 16;
    static constexpr int SP = DK + 8;       // padded LDS row of S^T (bf16)
    static_assert(NKT % NQT == 0 && NW <= 16, "query tiles split over waves");
    static_assert(NT % NW == 0 && TPW >= 1, "state tiles must split evenly over waves");
    static_assert(KBLK % 1024 == 0 && VBLK % 1024 == 0, "1 KiB direct-load units");
    static_assert(2 * KBLK + 2 * VBLK + QBLK + W * SP * 2 + 3 * BC * 4 <= 163840, "LDS budget");
    // XOR swizzle of the 16-byte chunks of a row: 16 consecutive rows read
    // at one logical chunk hit 16 different bank groups
    __device__ static int swz_k(int row) { return DK >= 128 ? (row & 15) : ((row >> 1) & 7); }
    __device__ static int swz_v(int row) { return (row >> 1) & 7; }
    __device__ static int koff(int row, int col) {  // byte offset of K~[row][col] (also Q~)
        return row * KROW + ((((col >> 3) ^ swz_k(row))) << 4) + (col & 7) * 2;
    }
    __device__ static int voff(int row, int col) {
        return row * VROW + ((((col >> 3) ^ swz_v(row))) << 4) + (col & 7) * 2;
    }
};

struct ChunkArgs {
    const uint16_t *q, *k, *v;  // Q~, K~ (already rotated), V
    uint16_t *o;
    const float *s_in;
    float *s_out;
    float2 *stats;  // [B*T*H][NS] (mean, M2) of each slice, when NS > 1
    int NS;         // slices per pair (dv / W)
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2 y = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, y);
}

__device__ __forceinline__ u32x4 ld16(const char *base, uint32_t off) {
    return *reinterpret_cast<const u32x4 *>(base + off);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (the LDS address is wave-uniform).
__device__ __forceinline__ void load_lds16(const void *gptr, void *lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)gptr,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// Keeps the scheduler from moving instructions across this point: used to
// issue the LDS fragment loads of the next k-step before the MFMAs of the
// current one.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// s_waitcnt with vmcnt = n and the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ s16x4 lds_tr_b(const char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)((__attribute__((address_space(3))) char *)(p)));
}

template <int DK, int BC>
__global__ __launch_bounds__((Cfg<DK, BC>::THREADS)) void chunk_mfma_kernel(MsrConst c, ChunkArgs a) {
    using C = Cfg<DK, BC>;
    // separate LDS objects for the two block buffers and the Q~ tile, so the
    // compiler can tell the direct loads into one from reads of another
    __shared__ __attribute__((aligned(16))) char Kb0[C::KBLK], Kb1[C::KBLK];
    __shared__ __attribute__((aligned(16))) char Vb0[C::VBLK], Vb1[C::VBLK];
    __shared__ __attribute__((aligned(16))) char Qs[C::QBLK];
    __shared__ __attribute__((aligned(16))) __bf16 St[W * C::SP];  // S_old^T
    __shared__ float dec[BC], xi[BC], zet[BC];  // s gamma^d, gamma^(j+1), s gamma^(BC-1-t)

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    // workgroup -> (pair, slice): the slices of one pair get ids equal mod 8,
    // i.e. run on the same XCD and share its L2 for the Q~ and K~ chunks.
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

    for (int t = tid; t < BC; t += C::THREADS) {
        dec[t] = c.scale * exp2f((float)t * lg);
        xi[t] = exp2f((float)(t + 1) * lg);
        zet[t] = c.scale * exp2f((float)(BC - 1 - t) * lg);
    }
    const float gb = exp2f((float)BC * lg);

    // uniform bases of this pair's rows; per-thread byte offsets fit 32 bits
    const uint32_t rowQK = (uint32_t)c.H * DK * 2;        // bytes between tokens of Q~, K~
    const uint32_t rowV = (uint32_t)c.H * c.dv * 2;       // bytes between tokens of V
    const char *qb = reinterpret_cast<const char *>(a.q + ((size_t)b * c.T * c.H + h) * DK);
    const char *kb = reinterpret_cast<const char *>(a.k + ((size_t)b * c.T * c.H + h) * DK);
    const char *vb = reinterpret_cast<const char *>(a.v + ((size_t)b * c.T * c.H + h) * c.dv + col0);

    // direct loads of 1 KiB units: unit u of a [rows][row bytes] tile whose
    // row r starts at global byte base + r * rstride; units go round-robin
    // over the waves
    auto dma_k = [&](const char *gbase, int tok0, char *dst, int nbytes) {
        for (int u = w; u < nbytes / 1024; u += C::NW) {
            const int byte = u * 1024 + lane * 16;
            const int row = byte / C::KROW, phys = (byte % C::KROW) >> 4;
            load_lds16(gbase + (uint32_t)(tok0 + row) * rowQK + (phys ^ C::swz_k(row)) * 16, dst + u * 1024);
        }
    };
    auto dma_v = [&](int tok0, char *dst) {
        for (int u = w; u < C::VBLK / 1024; u += C::NW) {
            const int byte = u * 1024 + lane * 16;
            const int row = byte / C::VROW, phys = (byte % C::VROW) >> 4;
            load_lds16(vb + (uint32_t)(tok0 + row) * rowV + (phys ^ C::swz_v(row)) * 16, dst + u * 1024);
        }
    };

    // query tiles of this wave: w and, with two, NKT-1-w (balances the causal work)
    int qtile[C::NQT];
    qtile[0] = w;
    if (C::NQT == 2) qtile[C::NQT - 1] = C::NKT - 1 - w;
    bf16x8 qreg[C::NQT][C::KS];  // this chunk's Q~ rows in MFMA operand layout
    auto take_q = [&](int t0) {
#pragma unroll
        for (int u = 0; u < C::NQT; ++u)
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int row = 16 * qtile[u] + l16, col = 32 * ks + 8 * g;
                if constexpr (C::QLDS)
                    qreg[u][ks] = *reinterpret_cast<const bf16x8 *>(Qs + C::koff(row, col));
                else
                    qreg[u][ks] = __builtin_bit_cast(bf16x8, ld16(qb, (uint32_t)(t0 + row) * rowQK + col * 2));
            }
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

    // finished, not yet stored outputs of the previous chunk
    uint32_t pend_o[C::NQT][C::CT][2];
    size_t pend_row[C::NQT];
    float2 pend_stat[C::NQT];
    const bool stats_out = a.NS > 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM);
    auto flush = [&]() {
#pragma unroll
        for (int u = 0; u < C::NQT; ++u) {
            uint16_t *dst = a.o + pend_row[u] * c.dv + col0 + 4 * g;
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) {
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 v2 = {pend_o[u][ct][0], pend_o[u][ct][1]};
                *reinterpret_cast<u32x2 *>(dst + ct * 16) = v2;
            }
            if (stats_out && g == 0) a.stats[pend_row[u] * a.NS + slice] = pend_stat[u];
        }
    };

    const int nchunks = c.T / BC;
    const int nblocks = nchunks * C::NB;
    write_st();
    if (nblocks > 0) {
        if constexpr (C::QLDS) dma_k(qb, 0, Qs, C::QBLK);
        dma_k(kb, 0, Kb0, C::KBLK);
        dma_v(0, Vb0);
    }

    f32x4 oacc[C::NQT][C::CT];
    // one key block: compute on (Kc, Vc) while the next block streams into (Kn, Vn)
    auto step = [&](int blk, const char *Kc, const char *Vc, char *Kn, char *Vn) {
        const int ci = blk / C::NB, kbi = blk % C::NB;
        const int t0 = ci * BC;
        // this block's direct loads (issued one step ago) are complete; the
        // Q~ tile of the next chunk, issued last in the previous step, may
        // still be in flight
        if (kbi == 1 && C::QLDS && ci + 1 < nchunks)
            wait_vm<0>();  // (nothing newer to spare at this point)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kbi == 0) {
            take_q(t0);
            if (ci > 0) flush();  // previous chunk's outputs
        }
        if (blk + 1 < nblocks) {
            dma_k(kb, (blk + 1) * C::KB, Kn, C::KBLK);
            dma_v((blk + 1) * C::KB, Vn);
        }
        if (kbi == 0) {
            // ---- O^T = (S_old^T Q~^T) xi for every query tile, then gamma^b S
            bf16x8 fa[C::CT], fb[C::CT];
#pragma unroll
            for (int u = 0; u < C::NQT; ++u)
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) oacc[u][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) fa[ct] = ld_lds8(St + (ct * 16 + l16) * C::SP + 8 * g);
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                if (ks + 1 < C::KS) {
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct)
                        fb[ct] = ld_lds8(St + (ct * 16 + l16) * C::SP + 32 * (ks + 1) + 8 * g);
                }
                sched_fence();
#pragma unroll
                for (int u = 0; u < C::NQT; ++u)
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct) oacc[u][ct] = mfma16(fa[ct], qreg[u][ks], oacc[u][ct]);
                sched_fence();
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) fa[ct] = fb[ct];
            }
#pragma unroll
            for (int u = 0; u < C::NQT; ++u) {
                const float x = xi[16 * qtile[u] + l16];
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) oacc[u][ct] = oacc[u][ct] * x;
            }
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = S[rt][ct] * gb;
        }
        // the next chunk's Q~ tile may be overwritten once every wave has
        // taken this chunk's rows (they all passed this step's barrier)
        if (C::QLDS && kbi == 1 && ci + 1 < nchunks) dma_k(qb, t0 + BC, Qs, C::QBLK);

        // ---- state update with this block's 32 tokens: S += K~^T (V zeta s)
        {
            const int tb = 8 * g;  // first token (within the block) of this lane group
            s16x4 vr[C::CPW][2], kr[C::RPW][2];
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct) {
                const int col = (cgw * C::CPW + ct) * 16 + 4 * (l16 & 3);
                vr[ct][0] = lds_tr_b(Vc + C::voff(tb + (l16 >> 2), col));
                vr[ct][1] = lds_tr_b(Vc + C::voff(tb + 4 + (l16 >> 2), col));
            }
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt) {
                const int col = (rgw * C::RPW + rt) * 16 + 4 * (l16 & 3);
                kr[rt][0] = lds_tr_b(Kc + C::koff(tb + (l16 >> 2), col));
                kr[rt][1] = lds_tr_b(Kc + C::koff(tb + 4 + (l16 >> 2), col));
            }
            float z[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = zet[kbi * C::KB + tb + e];
            bf16x8 bv[C::CPW];
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bv[ct][e] = static_cast<__bf16>(bf(vr[ct][0][e]) * z[e]);
                    bv[ct][4 + e] = static_cast<__bf16>(bf(vr[ct][1][e]) * z[4 + e]);
                }
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt) {
                const bf16x8 ak = cat(kr[rt][0], kr[rt][1]);
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = mfma16(ak, bv[ct], S[rt][ct]);
            }
        }

        // ---- intra-chunk part with this block's two 16-key tiles for the
        // query tiles that reach them (wave-uniform tests): P^T tiles with
        // decay, scale and causal mask in registers, packed as B operands,
        // then O^T += V^T P^T
        bool need[C::NQT];
        bool any = false;
#pragma unroll
        for (int u = 0; u < C::NQT; ++u) {
            need[u] = kbi * C::KB <= 16 * qtile[u] + 15;
            any = any || need[u];
        }
        if (any) {
            f32x4 acc[C::NQT][2];
#pragma unroll
            for (int u = 0; u < C::NQT; ++u) acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int v2 = 0; v2 < 2; ++v2)
                fa[v2] = *reinterpret_cast<const bf16x8 *>(Kc + C::koff(16 * v2 + l16, 8 * g));
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                if (ks + 1 < C::KS) {
#pragma unroll
                    for (int v2 = 0; v2 < 2; ++v2)
                        fb[v2] = *reinterpret_cast<const bf16x8 *>(Kc + C::koff(16 * v2 + l16, 32 * (ks + 1) + 8 * g));
                }
                sched_fence();
#pragma unroll
                for (int u = 0; u < C::NQT; ++u)
                    if (need[u]) {
#pragma unroll
                        for (int v2 = 0; v2 < 2; ++v2) acc[u][v2] = mfma16(fa[v2], qreg[u][ks], acc[u][v2]);
                    }
                sched_fence();
#pragma unroll
                for (int v2 = 0; v2 < 2; ++v2) fa[v2] = fb[v2];
            }
            s16x4 va[C::CT][2];
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct) {
                const int col = ct * 16 + 4 * (l16 & 3);
                va[ct][0] = lds_tr_b(Vc + C::voff(4 * g + (l16 >> 2), col));
                va[ct][1] = lds_tr_b(Vc + C::voff(16 + 4 * g + (l16 >> 2), col));
            }
#pragma unroll
            for (int u = 0; u < C::NQT; ++u) {
                if (!need[u]) continue;
                const int jq = 16 * qtile[u] + l16;
                bf16x8 pb;
#pragma unroll
                for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = kbi * C::KB + 16 * v2 + 4 * g + r;
                        const float x = (t <= jq) ? acc[u][v2][r] * dec[jq - t] : 0.f;
                        pb[4 * v2 + r] = static_cast<__bf16>(x);
                    }
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) oacc[u][ct] = mfma16(cat(va[ct][0], va[ct][1]), pb, oacc[u][ct]);
            }
        }

        if (kbi == C::NB - 1) {
            // ---- GroupNorm over each row (lanes l16, l16+16, +32, +48 share a query)
#pragma unroll
            for (int u = 0; u < C::NQT; ++u) {
                const int jq = 16 * qtile[u] + l16;
                float sum = 0.f;
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct)
                    sum += oacc[u][ct][0] + oacc[u][ct][1] + oacc[u][ct][2] + oacc[u][ct][3];
                sum += __shfl_xor(sum, 16, 64);
                sum += __shfl_xor(sum, 32, 64);
                const float mean = sum * (1.f / W);
                float m2 = 0.f;
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m2 += (oacc[u][ct][r] - mean) * (oacc[u][ct][r] - mean);
                m2 += __shfl_xor(m2, 16, 64);
                m2 += __shfl_xor(m2, 32, 64);
                float mu = 0.f, inv = 1.f;
                if (a.NS == 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM)) {
                    mu = mean;
                    inv = 1.f / sqrtf(m2 * (1.f / W) + c.eps);
                }
                // stored one chunk later (flush), so that waiting for the next
                // blocks' loads does not also wait for these stores
                pend_row[u] = ((size_t)b * c.T + t0 + jq) * c.H + h;
                pend_stat[u] = make_float2(mean, m2);
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) {
                    pend_o[u][ct][0] = pack_bf16x2((oacc[u][ct][0] - mu) * inv, (oacc[u][ct][1] - mu) * inv);
                    pend_o[u][ct][1] = pack_bf16x2((oacc[u][ct][2] - mu) * inv, (oacc[u][ct][3] - mu) * inv);
                }
            }
            // S_old^T was last read at this chunk's first block, before the
            // barrier of its second block
            write_st();
        }
    };
    for (int blk = 0; blk < nblocks; blk += 2) {
        step(blk, Kb0, Vb0, Kb1, Vb1);
        if (blk + 1 < nblocks) step(blk + 1, Kb1, Vb1, Kb0, Vb0);
    }
    if (nchunks > 0) flush();

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

// theta_shift of Q and K into bf16 copies, once per token and head: pair i
// of the token at position pos0 + t becomes (x0 c - x1 s, x1 c + x0 s) with
// (c, s) from the angle table; fp32 arithmetic.  8 channels per thread.
__global__ void rotate_qk_kernel(MsrConst c, const float2 *__restrict__ cs,
                                 const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                 uint16_t *__restrict__ qr, uint16_t *__restrict__ kr) {
    const int p8 = c.dk / 8;
    const size_t n = (size_t)c.B * c.T * c.H * p8;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int d8 = (int)(e % p8);
        const size_t row = e / p8;  // (b * T + t) * H + h
        const int t = (int)((row / c.H) % c.T);
        const float4 *cp = reinterpret_cast<const float4 *>(cs + (size_t)t * (c.dk / 2) + 4 * d8);
        const float4 c01 = cp[0], c23 = cp[1];
        const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
        const float ss[4] = {c01.y, c01.w, c23.y, c23.w};
        const u32x4 uq = reinterpret_cast<const u32x4 *>(q)[e];
        const u32x4 uk = reinterpret_cast<const u32x4 *>(k)[e];
        u32x4 oq, ok;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x0 = __uint_as_float(uq[i] << 16), x1 = __uint_as_float(uq[i] & 0xffff0000u);
            oq[i] = pack_bf16x2(x0 * cc[i] - x1 * ss[i], x1 * cc[i] + x0 * ss[i]);
            x0 = __uint_as_float(uk[i] << 16);
            x1 = __uint_as_float(uk[i] & 0xffff0000u);
            ok[i] = pack_bf16x2(x0 * cc[i] - x1 * ss[i], x1 * cc[i] + x0 * ss[i]);
        }
        reinterpret_cast<u32x4 *>(qr)[e] = oq;
        reinterpret_cast<u32x4 *>(kr)[e] = ok;
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
    const int grid = c.B * c.H * a.NS;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), 0, st, c, a);
    return hipGetLastError();
}

template <int DK>
hipError_t dispatch_bc(const MsrConst &c, const ChunkArgs &a, int chunk, hipStream_t st) {
    switch (chunk) {
    case 64: return launch_chunk<DK, 64>(c, a, st);
    case 128: return launch_chunk<DK, 128>(c, a, st);
    case 256: return launch_chunk<DK, 256>(c, a, st);
    default: return hipErrorNotSupported;
    }
}

struct MfmaPlan {
    size_t cs = 0, qr = 0, kr = 0, stats = 0, total = 0;
};

// workspace: [cos/sin table][Q~ bf16][K~ bf16][slice statistics]
MfmaPlan mfma_plan(const msr_problem *p) {
    MfmaPlan m;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t qk = (size_t)p->B * p->T * p->H * p->dk * 2;
    m.cs = 0;
    m.qr = up((size_t)p->T * (p->dk / 2) * sizeof(float2));
    m.kr = m.qr + up(qk);
    m.stats = m.kr + up(qk);
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
    if (chunk > p->T || p->T % chunk != 0) return false;
    // per-thread byte offsets within one batch row are 32-bit
    if ((uint64_t)p->T * p->H * (p->dk > p->dv ? p->dk : p->dv) * 2 >= (1ull << 32)) return false;
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
    const bool rotate = !(c.flags & MSR_FLAG_NO_ROTATE);
    ChunkArgs a;
    a.q = rotate ? reinterpret_cast<const uint16_t *>(wsb + m.qr) : static_cast<const uint16_t *>(Q);
    a.k = rotate ? reinterpret_cast<const uint16_t *>(wsb + m.kr) : static_cast<const uint16_t *>(K);
    a.v = static_cast<const uint16_t *>(V);
    a.o = static_cast<uint16_t *>(O);
    a.s_in = s_in;
    a.s_out = s_out;
    a.NS = p->dv / W;
    a.stats = a.NS > 1 ? reinterpret_cast<float2 *>(wsb + m.stats) : nullptr;

    hipError_t e = hipSuccess;
    if (rotate) {
        float2 *cs = reinterpret_cast<float2 *>(wsb + m.cs);
        const size_t ncs = (size_t)p->T * (p->dk / 2);
        size_t g = (ncs + 255) / 256;
        if (g > 65536) g = 65536;
        hipLaunchKernelGGL(angle_table_kernel, dim3((unsigned)g), dim3(256), 0, st, c, cs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const size_t n8 = (size_t)p->B * p->T * p->H * (p->dk / 8);
        g = (n8 + 255) / 256;
        if (g > 262144) g = 262144;
        hipLaunchKernelGGL(rotate_qk_kernel, dim3((unsigned)g), dim3(256), 0, st, c, cs,
                           static_cast<const uint16_t *>(Q), static_cast<const uint16_t *>(K),
                           reinterpret_cast<uint16_t *>(wsb + m.qr), reinterpret_cast<uint16_t *>(wsb + m.kr));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    main_kernel_begin(st);
    switch (p->dk) {
    case 64: e = dispatch_bc<64>(c, a, chunk, st); break;
    case 128: e = dispatch_bc<128>(c, a, chunk, st); break;
    case 256: e = dispatch_bc<256>(c, a, chunk, st); break;
    default: e = hipErrorNotSupported;
    }
    main_kernel_end(st);
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
