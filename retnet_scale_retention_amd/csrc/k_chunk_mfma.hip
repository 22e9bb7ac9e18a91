// k_chunk_mfma.hip -- bf16 matrix-core (MFMA) path of the chunkwise form.
//
// Per chunk i of b tokens (jsqmd.com "From RoPE to Retention" s4.3; aiqz.cc
// RetNet tutorial, "chunkwise recurrence"):
//   O_i = GN( (Q~_i K~_i^T (.) D) V_i + (Q~_i S_{i-1}) (.) xi )
//   S_i = gamma^b S_{i-1} + K~_i^T (V_i (.) zeta)
//
// Kernels, in launch order:
//   prep_kernel         per (pair, chunk), fully parallel (persistent
//                       workgroups, one per CU, where its tiles fill the
//                       LDS): rotates the chunk's Q and K rows, computes its
//                       masked, decayed scores P = (Q~ K~^T (.) D) s, and
//                       writes Q~, K~^T and P^T as MFMA operand fragments
//   chunk_mfma_kernel   the recurrence over the chunks, below (b <= 128:
//   / chunk_ws_kernel   its warp-specialised variant, which normalises rows
//                       spanning 2 to 8 slices itself by exchanging slice
//                       statistics between the slices' workgroups)
//   gn_finalize_kernel  GroupNorm when d_v spans several slices otherwise
//
// Fragments.  A 16x16x32 MFMA operand is 64 lanes x 8 bf16: lane 16 g + n
// holds row n, k-indices 8 g .. 8 g + 7.  prep_kernel stores each operand the
// chunk kernel reads from memory in exactly that order, 1 KiB per fragment,
// so every such load is one coalesced 16-byte-per-lane read into registers:
//   QF[pair][chunk][u][ks]  Q~, query rows 16 u.., d_k columns 32 ks..
//                           (B operand of the inter-chunk product)
//   KF[pair][chunk][rt][kb] (K~ zeta s)^T, d_k rows 16 rt.., tokens 32 kb..
//                           in the key order of PF below, with
//                           zeta_t s = s gamma^(b-1-t) and the rescale
//                           factor gamma^(-b j) of the chunk applied
//                           (A operand of the state update)
//   PF[pair][chunk][u][kb]  P^T, keys 32 kb.., query columns 16 u.., keys in
//                           the order {4g..4g+3, 16+4g..16+4g+3} of lane
//                           group g -- the values two 16x16 result tiles of
//                           P^T = K~ Q~^T leave in each lane
//                           (B operand of the value product)
//
// chunk_mfma_kernel.  A workgroup of NW waves (4, or 8 for b = 256) owns one (batch, head) pair
// and a slice of W = 64 value columns for the whole sequence; its fp32 state
// slice S[d_k][W] stays in MFMA accumulators for the entire run, split over
// the waves in 16x16 tiles.  Per chunk, behind one barrier:
//   - the chunk's V slice is in LDS (direct global->LDS loads issued one
//     chunk ahead into the other of two buffers);
//   - O^T = (S_old^T Q~^T) (.) xi, with S_old^T as bf16 in LDS;
//   - per 32-key block S^ += (K~ zeta s)^T V and O^T += V^T P^T, where S^ is
//     the state up to a power of gamma that changes only every m chunks
//     (rescale_period); V and V^T come from the gfx950 LDS transpose read
//     (ds_read_b64_tr_b16);
//   - GroupNorm of each output row over the slice (final when W == d_v,
//     otherwise (mean, M2) partials for gn_finalize_kernel);
//   - S_new^T as bf16 to the other LDS state buffer.
// Each register fragment is reloaded for a later block right after its last
// use, so the loads have most of a chunk to land.  Every wave issues the same
// loads in the same order each chunk, so one fixed vmcnt wait tells when the
// next V slice has landed.
#include <atomic>

#include "msr_chunk.hpp"
#include "msr_device.hpp"
#include "msr_mfma.hpp"

namespace msr {
// The call (its nonzero id) whose chunk kernel may wait on slice statistics
// and does not yet have all of its workgroups resident, or 0; one word per
// device, zero when the library loads.  A call that finds another owner runs
// without waiting (it stores raw rows, which the last workgroup of each
// (pair, segment) normalises from the slices' words).  The owner hands the
// word back once its last workgroup has started: from then on it completes
// on its own, so two calls that overlap on one GPU can never wait on each
// other's workgroups.
__device__ unsigned g_xg_owner;

// The exchange's counter words: 16, then one per (pair, segment); after
// them, from a 256-byte boundary, NEUTRAL_WORDS slice words that a call
// which does not wait reads in place of its row's words: mean 0 and an M2
// that makes the row's scale 1, so that it stores its rows unnormalised.
constexpr int NEUTRAL_WORDS = 128;
__host__ __device__ inline int xg_counter_words(int groups) { return (16 + groups + 63) / 64 * 64; }
}  // namespace msr

namespace {

using namespace msr;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int W = 64;      // value columns per workgroup slice
constexpr int FRAG = 512;  // bf16 elements per operand fragment

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read: within each 16-lane group, lane j points at 4
// consecutive bf16 of row r0 + j/4, columns c0 + 4 (j%4) ..; lane i then
// receives column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ s16x4 lds_tr(const void *p) {
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

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2 y = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, y);
}

__device__ __forceinline__ u32x4 ld16(const char *base, uint32_t off) {
    return *reinterpret_cast<const u32x4 *>(base + off);
}

__device__ __forceinline__ bf16x8 ldf(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// x[l] + x[l ^ 16] + x[l ^ 32] + x[l ^ 48], the same bits in every lane, with
// the gfx950 lane-swap instructions (permlane16_swap exchanges the odd 16-lane
// rows of its first operand with the even rows of its second, permlane32_swap
// the upper half of the first with the lower half of the second)
__device__ __forceinline__ float sum_lane_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (the LDS address is wave-uniform).
__device__ __forceinline__ void load_lds16(const void *gptr, void *lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)gptr,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// Keeps the scheduler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Keeps global-memory instructions (loads, stores, direct-to-LDS loads) in
// program order across this point; ALU, MFMA and LDS instructions may still
// move across it.
__device__ __forceinline__ void vmem_fence() { __builtin_amdgcn_sched_barrier(0x078F); }

// s_waitcnt with vmcnt = n and the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int DK, int BC>
struct Cfg {
    static constexpr int NKT = BC / 16;        // 16-token tiles per chunk
    static constexpr int NB = BC / 32;         // 32-key blocks per chunk
    static constexpr int KS = DK / 32;         // 32-wide k-steps over d_k
    static constexpr int RT = DK / 16;         // 16-row tiles of d_k
    static constexpr int NW = BC == 256 ? 8 : 4;  // waves per workgroup
    static constexpr int THREADS = NW * 64;
    static constexpr int NQT = NKT / NW;       // query tiles per wave
    static constexpr int CT = W / 16;          // value column tiles
    static constexpr int TPW = RT * CT / NW;   // 16x16 state tiles per wave
    static constexpr int CPW = TPW < CT ? TPW : CT;  // ... in this many column tiles
    static constexpr int RPW = TPW / CPW;            // ... and row tiles
    static constexpr int CG = CT / CPW;              // column groups of waves
    static constexpr int R = NB <= 4 ? NB : 1; // key blocks of K~^T / P^T fragments held in registers
    static constexpr int KROW = DK * 2;        // bytes per K~ row in LDS (prep_kernel)
    // prep_kernel stages Q~ in LDS next to K~ when both fit (1024 threads
    // when they need more than half of the LDS, so that a CU still holds 16
    // waves); otherwise Q~ goes straight to its fragments and the scores read
    // it back from there
    static constexpr bool QSTAGE = 2 * BC * KROW + 2 * BC * 4 <= 163840;
    static constexpr int PREP_NT = QSTAGE && 2 * BC * KROW > 81920 ? 1024 : 512;
    // prep_kernel's LDS tiles leave room for one workgroup per CU: its
    // workgroups are then persistent (one per CU, several chunks each)
    static constexpr bool PREP_PERSIST = (QSTAGE ? 2 : 1) * BC * KROW > 81920;
    static constexpr int VROW = W * 2;         // bytes per V row in LDS
    static constexpr int VTILE = BC * VROW;    // bytes of a chunk's V slice
    static constexpr int NV = VTILE / 1024 / NW;  // direct-load units per wave per chunk
    static constexpr int SP = DK + 8;          // padded LDS row of S^T (bf16)
    // memory operations each wave issues per chunk after the next V slice:
    // per block, its K~^T and P^T fragments and a share of the next chunk's
    // Q~ fragments.  The V loads go first (during the inter-chunk product)
    // when the count allows, else right before block KBV.
    static constexpr int NQ = NQT * KS;
    static constexpr int PER_BLK = RPW + NQT;
    __host__ __device__ static constexpr int qpart0(int kb) { return kb * NQ / NB; }  // first Q~ load of block kb
    __host__ __device__ static constexpr int after_v(int kbv) { return (NB - kbv) * PER_BLK + NQ - qpart0(kbv); }
    __host__ __device__ static constexpr int first_kbv() {
        int kb = 0;
        while (kb < NB && after_v(kb) > 63) ++kb;
        return kb;
    }
    static constexpr bool V_FIRST = after_v(0) <= 63;
    static constexpr int KBV = V_FIRST ? 0 : first_kbv();
    static constexpr int VWAIT = after_v(KBV);
    // state-only pass: V first, then only the K~^T fragments of every block
    static constexpr int VWAIT_SO = NB * RPW;
    static_assert(VWAIT_SO <= 63, "vmcnt range");
    static_assert(NQT >= 1 && RPW >= 1 && NV >= 1 && (NW / CG) * RPW == RT && CG * CPW == CT, "shape");
    static_assert(VWAIT <= 63 && KBV < NB, "vmcnt range");
    static_assert(2 * VTILE + 2 * W * SP * 2 + 2 * BC * 4 <= 163840, "LDS budget (chunk kernel)");
    // query tiles of wave w: w, 2 NW - 1 - w, 2 NW + w, 4 NW - 1 - w, ... (equal causal work)
    __device__ static int qtile(int w, int i) {
        return (i & 1) ? 2 * NW * (i / 2 + 1) - 1 - w : 2 * NW * (i / 2) + w;
    }
    // XOR swizzle of the 16-byte chunks of a row: 16 consecutive rows read at
    // one logical chunk land in different bank groups
    __device__ static int swz_k(int row) { return DK >= 128 ? (row & 15) : ((row >> 1) & 7); }
    __device__ static int swz_v(int row) { return (row >> 1) & 7; }
    __device__ static int koff(int row, int col) {  // byte offset of K~[row][col]
        return row * KROW + ((((col >> 3) ^ swz_k(row))) << 4) + (col & 7) * 2;
    }
    __device__ static int voff(int row, int col) {
        return row * VROW + ((((col >> 3) ^ swz_v(row))) << 4) + (col & 7) * 2;
    }
};

// Per (pair, chunk): rotation of the chunk's Q and K rows (theta_shift,
// jsqmd.com s2: pair i of the token at position p becomes
// (x0 c - x1 s, x1 c + x0 s) with c, s = cos, sin of p theta_i; fp32
// arithmetic, rounded to bf16), then the chunk's scores
//   P[j][t] = s gamma^(j-t) (q~_j . k~_t) for t <= j, else 0
// with the decay and the causal mask applied in registers.  Writes the QF,
// KF and PF fragments described at the top of the file.
//
// Rotation: thread (c8, rg) handles channels 8 c8 .. 8 c8 + 7 (4 pairs) of a
// run of RPT consecutive rows.  The angles of the run's first row come from
// rot_cos_sin (fp64 quarter-turn reduction); each next row multiplies (cos, sin) by
// (cos theta_i, sin theta_i) -- the angle-addition formula, a few ulp of
// drift over at most 16 rows.  Q~ goes straight to its fragments in global
// memory, K~ of the chunk to LDS; the score products read Q~ back from the
// fragments (visible to the workgroup after the barrier).  P^T fragments of
// key blocks a query tile does not reach are not written (the chunk kernel
// loads but never uses them).
//
// PAR (parallel form, b = 64): no scores; K~ also goes to fragments in the
// Q~ layout (kq, the A operand of the parallel kernel's score products), and
// the KF fragments carry s gamma^(T-1-t) for the state sum
// S_out = gamma^T S_in + sum_t gamma^(T-1-t) k~_t^T v_t.
//
// SPLIT: q and k come with low parts qlo, klo of the same layout (two-term
// bf16 splits of more precise operands); the scores then take
// hi.hi + lo.hi + hi.lo, the lo fragments read straight from global memory.
// Everything else uses the hi parts.
//
// QPERM: the QF fragments hold their d_k columns in the order
// {4g..4g+3, 16+4g..16+4g+3} of lane group g within each 32-column step --
// the rows two 16x16 state tiles leave in each lane, so that a kernel
// holding the state in MFMA accumulators can feed it to the inter-chunk
// product without a transpose (k_chunk_wide.hip).
template <int DK, int BC, bool PAR, bool SPLIT = false, bool QPERM = false>
__global__ __launch_bounds__((Cfg<DK, BC>::PREP_NT)) void prep_kernel(MsrConst c, const uint16_t *__restrict__ q,
                                                                  const uint16_t *__restrict__ k,
                                                                  uint16_t *__restrict__ qf, uint16_t *__restrict__ kf,
                                                                  uint16_t *__restrict__ pf, uint16_t *__restrict__ kq,
                                                                  const uint16_t *__restrict__ qlo = nullptr,
                                                                  const uint16_t *__restrict__ klo = nullptr,
                                                                  unsigned long long *__restrict__ xz = nullptr,
                                                                  int xns = 0, unsigned *__restrict__ xtick = nullptr,
                                                                  unsigned xid = 0, int xng = 0) {
    using C = Cfg<DK, BC>;
    constexpr int NT = C::PREP_NT, PW = NT / 64;  // threads, waves
    constexpr int C8 = DK / 8;                    // 16-byte channel groups per row
    constexpr int RG = NT / C8;                   // row runs
    constexpr int RPT = BC / RG;                  // rows per run
    constexpr bool QS = C::QSTAGE;
    static_assert(RPT >= 1 && RG * RPT == BC, "row runs");
    static_assert(!QPERM || (QS && !PAR), "QPERM fragments are formed from the staged Q~ tile");
    static_assert((QS ? 2 : 1) * BC * C::KROW + 2 * BC * 4 <= 163840, "LDS budget (prep kernel)");
    __shared__ __attribute__((aligned(16))) char Ks[BC * C::KROW];            // K~, swizzled rows
    __shared__ __attribute__((aligned(16))) char Qs[QS ? BC * C::KROW : 16];  // Q~, the same layout
    __shared__ float dec[BC], zet[BC];  // s gamma^d, s gamma^(BC-1-t)
    __shared__ float2 step[DK / 2];     // cos and sin of theta_i: the angle step from row to row

    const int nch = c.T / BC;
    const int nblk = c.B * c.H * nch;  // (pair, chunk) blocks
    const int ld = c.ldqk ? c.ldqk : DK;            // Q, K may be column slices of wider rows
    const uint32_t rowQK = (uint32_t)c.H * ld * 2;  // bytes between tokens of Q, K
    const bool rv = c.revqk != 0;
    // byte offset of the chunk's row r from its first source token's row
    auto roff = [&](int r) { return (uint32_t)(rv ? BC - 1 - r : r) * rowQK; };
    // element offset of (pair, chunk) block blk's first source token row
    auto block_base = [&](int blk) {
        const int pr = blk / nch, cj = blk % nch;
        const int tlo = rv ? c.T - (cj + 1) * BC : cj * BC;  // lowest source token of the chunk
        return (((size_t)(pr / c.H) * c.T + (size_t)tlo) * c.H + pr % c.H) * ld;
    };
    // Workgroup w takes blocks w, w + gridDim.x, ...: one block each unless
    // the tiles leave room for a single workgroup per CU (PREP_PERSIST), where
    // the grid holds one workgroup per CU.  A thread holds its rotation rows
    // of Q and K in registers; in a persistent workgroup, when they are few
    // (PREFETCH), the next block's rows are loaded as soon as the current
    // block's rotation has consumed them, so the loads overlap its fragment
    // and score stage instead of following it.
    constexpr bool PREFETCH = C::PREP_PERSIST && RPT <= 4;
    const int c8 = (int)threadIdx.x % C8, r0 = ((int)threadIdx.x / C8) * RPT;
    u32x4 xq[RPT], xk[RPT];
    auto load_rows = [&](int blk) {
        const char *qr = reinterpret_cast<const char *>(q + block_base(blk));
        const char *kr = reinterpret_cast<const char *>(k + block_base(blk));
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            xq[j] = ld16(qr, roff(r0 + j) + c8 * 16);
            xk[j] = ld16(kr, roff(r0 + j) + c8 * 16);
        }
    };
    const bool rot = !(c.flags & MSR_FLAG_NO_ROTATE);
    if (rot) {
        for (int i = threadIdx.x; i < DK / 2; i += NT) {
            float cs, sn;
            rot_cos_sin(1, c.theta[i], cs, sn);
            step[i] = float2{cs, sn};
        }
    }
    __syncthreads();
  auto body = [&](int blk) __attribute__((always_inline)) {
    if (!PREFETCH) load_rows(blk);
    // (persistent: lane-dependent values are formed again from an opaque copy
    // of the thread index in every block, rather than kept live across the loop)
    int tid_r = threadIdx.x;
    if constexpr (C::PREP_PERSIST) asm volatile("" : "+v"(tid_r));
    const int tid = tid_r, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int pair = blk / nch, ci = blk % nch;
    const int b = pair / c.H, h = pair % c.H;
    const float lg = c.log2g[h];
    if (xz) {
        // the chunk kernel's GroupNorm exchange words of this block (BC xns,
        // contiguous), and its ticket counters, start at zero
        u32x4 *xr = reinterpret_cast<u32x4 *>(xz + (size_t)blk * BC * xns);
        for (int i = tid; i < BC * xns / 2; i += NT) xr[i] = u32x4{0u, 0u, 0u, 0u};
        // and decides whether the chunk kernel may wait on the slices' words:
        // mode 1 if this call claims the device's exchange, 2 if another
        // call holds it (a replay of this same call included) or the call
        // has no id.  Words 0-7 are the ticket queues, which carry the mode
        // in their top bit (one atomic gives a workgroup its ticket and the
        // mode), word 8 the mode, word 9 the count of queues whose
        // workgroups have all started (the chunk kernel hands the claim back
        // at the last), words 16 .. 16 + xng - 1 the finished workgroups of
        // each (pair, segment) in mode 2.
        if (blk == 0) {
            if (tid == 0) {
                unsigned prev = 1u;  // (no id: as if claimed)
                if (xid) {
                    prev = 0u;
                    __hip_atomic_compare_exchange_strong(&g_xg_owner, &prev, xid, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
                }
                const unsigned md = prev == 0u ? 1u : 2u;
                for (int q = 0; q < 8; ++q) xtick[q] = md == 2u ? 0x80000000u : 0u;
                xtick[8] = md;
            }
            for (int i = 9 + tid; i < 16 + xng; i += NT) xtick[i] = 0u;
            // neutral words: each slice M2 = (1 - eps) d_v / NS, so the row's
            // variance plus eps is 1
            unsigned long long *xn = reinterpret_cast<unsigned long long *>(xtick + xg_counter_words(xng));
            const float m2n = (1.f - c.eps) * (float)c.dv / (float)xns;
            for (int i = tid; i < NEUTRAL_WORDS; i += NT)
                xn[i] = (unsigned long long)(__float_as_uint(m2n) | 0x80000000u) << 32;
        }
    }
    for (int t = tid; t < BC; t += NT) {
        dec[t] = c.scale * exp2f((float)t * lg);
        if (PAR)  // s gamma^(T-1-t) for absolute token t
            zet[t] = c.scale * exp2f((float)(c.T - 1 - ci * BC - t) * lg);
        else  // s gamma^(BC-1-t) gamma^(-BC j), j = chunk index mod the rescale period
            zet[t] = c.scale * exp2f((float)(BC - 1 - t - BC * (ci % rescale_period(lg, BC))) * lg);
    }

    const size_t base = block_base(blk);

    uint16_t *qfo = qf + (size_t)blk * (C::NKT * C::KS * FRAG);
    {  // ---- rotation: Q~ into LDS (or to its fragments), K~ into LDS
        float cc[4] = {1.f, 1.f, 1.f, 1.f}, ss[4] = {0.f, 0.f, 0.f, 0.f}, c1[4], s1[4];
        if (rot) {
            const int64_t p0 = row_pos0(c, b) + (int64_t)ci * BC + r0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rot_cos_sin(p0, c.theta[4 * c8 + i], cc[i], ss[i]);
                const float2 st = step[4 * c8 + i];
                c1[i] = st.x;
                s1[i] = st.y;
            }
        }
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            u32x4 yq, yk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x0 = __uint_as_float(xq[j][i] << 16), x1 = __uint_as_float(xq[j][i] & 0xffff0000u);
                yq[i] = pack_bf16x2(x0 * cc[i] - x1 * ss[i], x1 * cc[i] + x0 * ss[i]);
                x0 = __uint_as_float(xk[j][i] << 16);
                x1 = __uint_as_float(xk[j][i] & 0xffff0000u);
                yk[i] = pack_bf16x2(x0 * cc[i] - x1 * ss[i], x1 * cc[i] + x0 * ss[i]);
            }
            // fragment (u, ks) = (row / 16, c8 / 4), lane 16 (c8 % 4) + row % 16
            const int row = r0 + j;
            const size_t fo = (size_t)((row >> 4) * C::KS + (c8 >> 2)) * FRAG + (16 * (c8 & 3) + (row & 15)) * 8;
            if (QS)
                *reinterpret_cast<u32x4 *>(Qs + C::koff(row, c8 * 8)) = rot ? yq : xq[j];
            else
                *reinterpret_cast<u32x4 *>(qfo + fo) = rot ? yq : xq[j];
            if (PAR) *reinterpret_cast<u32x4 *>(kq + (size_t)blk * (C::NKT * C::KS * FRAG) + fo) = rot ? yk : xk[j];
            *reinterpret_cast<u32x4 *>(Ks + C::koff(row, c8 * 8)) = rot ? yk : xk[j];
            if (rot && j + 1 < RPT) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float cn = cc[i] * c1[i] - ss[i] * s1[i];
                    ss[i] = ss[i] * c1[i] + cc[i] * s1[i];
                    cc[i] = cn;
                }
            }
        }
    }
    if (PREFETCH && blk + (int)gridDim.x < nblk) load_rows(blk + gridDim.x);
    __syncthreads();

    // ---- Q~ fragments from LDS, one whole fragment per store.  For the
    // chunkwise form they carry the row factor of the inter-chunk term,
    //   xi_j gamma^(BC ph) = gamma^(j + 1 + BC ph),  ph = (ci - 1) mod m (0 for ci = 0),
    // the phase m of the state the chunk kernel carries on entering chunk ci
    // (rescale_period), so that its product with that state is the term itself.
    if (QS) {
        const int ph = ci == 0 ? 0 : (ci - 1) % rescale_period(lg, BC);
        for (int f = w; f < C::NKT * C::KS; f += PW) {
            const int u = f / C::KS, ks = f % C::KS, row = 16 * u + l16;
            u32x4 x;
            if constexpr (QPERM) {
                const u32x2 lo = *reinterpret_cast<const u32x2 *>(Qs + C::koff(row, 32 * ks + 4 * g));
                const u32x2 hi = *reinterpret_cast<const u32x2 *>(Qs + C::koff(row, 32 * ks + 16 + 4 * g));
                x = u32x4{lo[0], lo[1], hi[0], hi[1]};
            } else {
                x = ld16(Qs, C::koff(row, 32 * ks + 8 * g));
            }
            u32x4 y = x;
            if (!PAR) {
                const float fq = exp2f((float)(row + 1 + BC * ph) * lg);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[i] = pack_bf16x2(__uint_as_float(x[i] << 16) * fq, __uint_as_float(x[i] & 0xffff0000u) * fq);
            }
            *reinterpret_cast<u32x4 *>(qfo + (size_t)f * FRAG + lane * 8) = y;
        }
    }

    // ---- (K~ zeta s)^T fragments: lane (n, g) of fragment (rt, kb) holds
    // K~[t][16 rt + n] s gamma^(BC-1-t) gamma^(-BC j) for t = 32 kb + 4 g + e
    // and t = 32 kb + 16 + 4 g + e (e = 0..3): the key order of the P^T
    // fragments, so that one transposed read of V serves both products
    uint16_t *kfo = kf + (size_t)blk * (C::RT * C::NB * FRAG) + lane * 8;
    for (int f = w; f < C::RT * C::NB; f += PW) {
        const int rt = f / C::NB, kb = f % C::NB;
        const int row = 32 * kb + 4 * g + (l16 >> 2), col = 16 * rt + 4 * (l16 & 3);
        const s16x4 lo = lds_tr(Ks + C::koff(row, col)), hi = lds_tr(Ks + C::koff(row + 16, col));
        bf16x8 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = static_cast<__bf16>(bf(lo[e]) * zet[32 * kb + 4 * g + e]);
            x[4 + e] = static_cast<__bf16>(bf(hi[e]) * zet[32 * kb + 16 + 4 * g + e]);
        }
        *reinterpret_cast<bf16x8 *>(kfo + (size_t)f * FRAG) = x;
    }

    // ---- P^T = K~ Q~^T for every (query tile u, 32-key block kb) the tile
    // reaches (32 kb <= 16 u + 15, i.e. kb <= u / 2), masked, decayed and
    // scaled.  The items, in (u, kb) order, are dealt to all the waves in turn
    // (at most two per wave at the 7B shape's 20 items and 16 waves).
    if (!PAR) {
        constexpr int NI = [] {
            int n = 0;
            for (int u = 0; u < C::NKT; ++u) n += u / 2 + 1;
            return n;
        }();
        uint16_t *pfo = pf + (size_t)blk * (C::NKT * C::NB * FRAG) + lane * 8;
        for (int it = w; it < NI; it += PW) {
            int u = 0, kb = it;  // (uniform)
            while (kb > u / 2) {
                kb -= u / 2 + 1;
                ++u;
            }
            f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                bf16x8 ka[2];
#pragma unroll
                for (int v2 = 0; v2 < 2; ++v2)
                    ka[v2] = *reinterpret_cast<const bf16x8 *>(Ks + C::koff(32 * kb + 16 * v2 + l16, 32 * ks + 8 * g));
                const bf16x8 qb = QS ? __builtin_bit_cast(bf16x8, ld16(Qs, C::koff(16 * u + l16, 32 * ks + 8 * g)))
                                     : ldf(qfo + (size_t)(u * C::KS + ks) * FRAG + lane * 8);
#pragma unroll
                for (int v2 = 0; v2 < 2; ++v2) acc[v2] = mfma16(ka[v2], qb, acc[v2]);
                if constexpr (SPLIT) {
                    const char *ql = reinterpret_cast<const char *>(qlo + base);
                    const char *kl = reinterpret_cast<const char *>(klo + base);
                    const bf16x8 qlb =
                        __builtin_bit_cast(bf16x8, ld16(ql, roff(16 * u + l16) + (32 * ks + 8 * g) * 2));
#pragma unroll
                    for (int v2 = 0; v2 < 2; ++v2) {
                        const bf16x8 kla = __builtin_bit_cast(
                            bf16x8, ld16(kl, roff(32 * kb + 16 * v2 + l16) + (32 * ks + 8 * g) * 2));
                        acc[v2] = mfma16(kla, qb, acc[v2]);
                        acc[v2] = mfma16(ka[v2], qlb, acc[v2]);
                    }
                }
            }
            const int jq = 16 * u + l16;
            bf16x8 pb;
#pragma unroll
            for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 32 * kb + 16 * v2 + 4 * g + r;
                    pb[4 * v2 + r] = static_cast<__bf16>((t <= jq) ? acc[v2][r] * dec[jq - t] : 0.f);
                }
            *reinterpret_cast<bf16x8 *>(pfo + (size_t)(u * C::NB + kb) * FRAG) = pb;
        }
    }
    if constexpr (C::PREP_PERSIST) __syncthreads();  // every wave is done with Ks, Qs, dec and zet of this block
  };
    if constexpr (C::PREP_PERSIST) {
        if (PREFETCH && (int)blockIdx.x < nblk) load_rows(blockIdx.x);
        for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) body(blk);
    } else {
        body(blockIdx.x);
    }
}

// Segments.  When the (pair, slice) workgroups are too few to fill the GPU,
// each pair's chunks are split into nseg segments of seglen chunks.  The
// state-only instantiation (SO) runs segments 0 .. nseg-2 from a zero state
// with only the state update and writes each end state E_g (and sets s_in
// aside in the unused slot of segment nseg-1); the full
// instantiation then starts segment g from
//   S_in(g) = gamma^(b seglen) S_in(g-1) + E_(g-1),  S_in(0) = s_in
// (the chunkwise recurrence regrouped by segments) and writes its outputs.
template <int DK, int BC, bool SO>
__global__ __launch_bounds__((Cfg<DK, BC>::THREADS)) void chunk_mfma_kernel(MsrConst c, ChunkArgs a) {
    using C = Cfg<DK, BC>;
    // separate LDS objects for the two V buffers, so the compiler can tell the
    // direct loads into one from reads of the other
    __shared__ __attribute__((aligned(16))) char Vb0[C::VTILE], Vb1[C::VTILE];
    __shared__ __attribute__((aligned(16))) __bf16 St0[W * C::SP], St1[W * C::SP];  // S_old^T
    __shared__ float xi[BC];  // gamma^(j+1)

    // the wave index is uniform across the wave: keep it (and what derives
    // from it) in scalar registers
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    // workgroup -> (pair, segment, slice): the slices of one (pair, segment)
    // get ids equal mod 8, i.e. run on the same XCD and share its L2 for the
    // fragments they all read
    const int npairs = c.B * c.H;
    int pair, seg, slice;
    {
        const int id = blockIdx.x, nps = npairs * a.nseg;
        int ps;
        if (nps % 8 == 0) {
            const int xcd = id & 7, j = id >> 3;
            ps = (j / a.NS) * 8 + xcd;
            slice = j % a.NS;
        } else {
            ps = id / a.NS;
            slice = id % a.NS;
        }
        pair = ps / a.nseg;
        seg = ps % a.nseg;
    }
    const int col0 = slice * W;
    if (SO && !a.par && seg == a.nseg - 1) {
        // The last segment's end state is not needed.  Its slot holds a copy
        // of this slice of s_in instead, which the full pass reads: the full
        // pass may then write s_out over s_in in any workgroup order.
        const size_t sb = (size_t)pair * DK * c.dv + col0;
        float *dst = a.segE + (size_t)pair * a.nseg * DK * c.dv + (size_t)seg * DK * c.dv + col0;
        for (int i = tid; i < DK * W; i += C::THREADS) {
            const size_t o = (size_t)(i / W) * c.dv + i % W;
            dst[o] = a.s_in ? a.s_in[sb + o] : 0.f;
        }
        return;
    }
    const int i0 = seg * a.seglen, i1 = i0 + a.seglen;  // this workgroup's chunks
    const int b = pair / c.H, h = pair % c.H;
    const float lg = c.log2g[h];
    for (int t = tid; t < BC; t += C::THREADS) xi[t] = exp2f((float)(t + 1) * lg);
    // (the parallel form's KF fragments carry the whole decay: no rescaling)
    const int period = a.par ? (1 << 30) : rescale_period(lg, BC);
    // the carried S^ is S gamma^(-BC ph); entering chunk i0 it has the phase
    // of chunk i0 - 1
    int ph = i0 == 0 ? 0 : (i0 - 1) % period;

    const int nch = c.T / BC;
    const size_t pc0 = (size_t)pair * nch;  // (pair, chunk 0) index of the fragments
    // uniform fragment bases; each lane adds its 16-byte offset
    const uint16_t *qfb = a.qf + pc0 * (C::NKT * C::KS * FRAG);
    const uint16_t *kfb = a.kf + pc0 * (C::RT * C::NB * FRAG);
    const uint16_t *pfb = a.pf + pc0 * (C::NKT * C::NB * FRAG);
    const uint32_t loff = lane * 16;
    auto ldfrag = [&](const uint16_t *fb, size_t frag) {
        return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(fb + frag * FRAG) + loff);
    };
    const uint32_t rowV = (uint32_t)c.H * c.dv * 2;  // bytes between tokens of V
    const char *vb = reinterpret_cast<const char *>(a.v + ((size_t)b * c.T * c.H + h) * c.dv + col0);

    int qt[C::NQT];
#pragma unroll
    for (int i = 0; i < C::NQT; ++i) qt[i] = C::qtile(w, i);
    // state tiles of this wave: row tiles rbase.., column tiles cbase..
    const int rbase = (w / C::CG) * C::RPW, cbase = (w % C::CG) * C::CPW;

    // ---- loads; indices past the last chunk are clamped to it, so every
    // wave issues the same operations every chunk
    auto dma_v_unit = [&](int ci, int i, char *dst) {
        ci = ci < nch ? ci : nch - 1;
        const int unit = i * C::NW + w;
        const int byte = unit * 1024 + lane * 16;
        const int row = byte / C::VROW, phys = (byte % C::VROW) >> 4;
        load_lds16(vb + (uint32_t)(ci * BC + row) * rowV + (phys ^ C::swz_v(row)) * 16, dst + unit * 1024);
    };
    auto dma_v = [&](int ci, char *dst) {
#pragma unroll
        for (int i = 0; i < C::NV; ++i) dma_v_unit(ci, i, dst);
    };
    bf16x8 qr[C::NQT][C::KS];   // Q~ fragments of the current chunk
    bf16x8 kr[C::RPW][C::R];    // K~^T fragments, slot kb % R
    bf16x8 pr[C::NQT][C::R];    // P^T fragments, slot kb % R
    // Q~ fragments f0 .. f1 - 1 (f = u KS + ks) of chunk ci
    auto load_q = [&](int ci, int f0, int f1) {
        ci = ci < nch ? ci : nch - 1;
#pragma unroll
        for (int f = 0; f < C::NQ; ++f)
            if (f >= f0 && f < f1)
                qr[f / C::KS][f % C::KS] = ldfrag(qfb, (size_t)(ci * C::NKT + qt[f / C::KS]) * C::KS + f % C::KS);
    };
    // K~^T and P^T fragments of block kb of chunk ci into slot kb % R
    auto load_kp_k = [&](int ci, int kb) {
        ci = ci < nch ? ci : nch - 1;
#pragma unroll
        for (int rt = 0; rt < C::RPW; ++rt)
            kr[rt][kb % C::R] = ldfrag(kfb, (size_t)(ci * C::RT + rbase + rt) * C::NB + kb);
    };
    auto load_kp_p = [&](int ci, int kb) {
        ci = ci < nch ? ci : nch - 1;
#pragma unroll
        for (int u = 0; u < C::NQT; ++u)
            pr[u][kb % C::R] = ldfrag(pfb, (size_t)(ci * C::NKT + qt[u]) * C::NB + kb);
    };
    // L2 prefetch of the pair's fragment lines of the next chunk, each slice
    // its 1/NS share, one dword per 128-byte line, in the full pass with 8 or
    // more slices per pair (as in chunk_ws_kernel; 7B-shaped layer at b = 256:
    // 0.581 -> 0.566 ms per call).  It is issued right after the chunk's
    // barrier, before the chunk's V loads, so the fixed wait counts after
    // the V loads are unchanged; the dword is kept live until the next
    // prefetch, a chunk later.
    constexpr int QFB = C::NKT * C::KS * FRAG * 2, KFB = C::RT * C::NB * FRAG * 2, PFB = C::NKT * C::NB * FRAG * 2;
    constexpr int NL = (QFB + KFB + PFB) / 128;  // fragment lines per chunk
    const int lps = (NL + a.NS - 1) / a.NS;     // ... per slice
    const int pl = slice * lps + w * 64 + lane;  // this lane's line
    const bool pf_on = !SO && a.NS >= 8 && w * 64 + lane < lps && pl < NL;
    uint32_t pfv = 0u;
    auto prefetch = [&](int cj) {
        cj = cj < nch ? cj : nch - 1;
        const char *p = pl < QFB / 128   ? reinterpret_cast<const char *>(qfb) + (size_t)cj * QFB + pl * 128
                        : pl < (QFB + KFB) / 128
                            ? reinterpret_cast<const char *>(kfb) + (size_t)cj * KFB + (pl - QFB / 128) * 128
                            : reinterpret_cast<const char *>(pfb) + (size_t)cj * PFB + (pl - (QFB + KFB) / 128) * 128;
        asm volatile("" ::"v"(pfv));
        if (pf_on) pfv = *reinterpret_cast<const uint32_t *>(p);
    };

    // ---- state tiles: d_k rows (rbase + rt) 16 + 4 g + r, columns (cbase + ct) 16 + l16
    f32x4 S[C::RPW][C::CPW];
    const size_t sbase = (size_t)pair * DK * c.dv + col0;
    // E_g of this pair: segE + ((pair nseg + g) DK + row) dv + col0 + col
    const size_t ebase = (size_t)pair * a.nseg * DK * c.dv + col0;
    // the incoming state: with segments, the copy the state-only pass made
    const float *sin_p = a.nseg > 1 ? a.segE + ebase + (size_t)(a.nseg - 1) * DK * c.dv
                                    : (a.s_in ? a.s_in + sbase : nullptr);
    {
        const float gseg = exp2f((float)(BC * a.seglen) * lg);  // gamma^(b seglen)
        const float f0 = exp2f(-(float)(BC * ph) * lg);         // to the carried scale
#pragma unroll
        for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = (rbase + rt) * 16 + 4 * g + r, col = (cbase + ct) * 16 + l16;
                    float x = 0.f;
                    if (!SO)
                        x = sin_p ? sin_p[(size_t)row * c.dv + col] : 0.f;
                    else if (a.par && a.s_in)  // gamma^T s_in
                        x = a.s_in[sbase + (size_t)row * c.dv + col] * exp2f((float)c.T * lg);
                    S[rt][ct][r] = x;
                }
        if (!SO) {
            // earlier segments' end states
            fold_segments<64>(S, a.segE + ebase, (size_t)DK * c.dv, seg, gseg, [&](int rt, int ct, int r) {
                return (size_t)((rbase + rt) * 16 + 4 * g + r) * c.dv + (cbase + ct) * 16 + l16;
            });
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = S[rt][ct] * f0;
        }
    }
    auto write_st = [&](__bf16 *St) {
#pragma unroll
        for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct) {
                const int row = (rbase + rt) * 16 + 4 * g, col = (cbase + ct) * 16 + l16;
                bf16x4 v4;
#pragma unroll
                for (int r = 0; r < 4; ++r) v4[r] = static_cast<__bf16>(S[rt][ct][r]);
                *reinterpret_cast<bf16x4 *>(St + col * C::SP + row) = v4;
            }
    };

    // finished outputs of the previous chunk, stored during the next chunk.
    // Before the first chunk they hold zeros for chunk 0's rows, which the
    // real values overwrite later (stores of one wave to one address stay in
    // order), so that every chunk issues the same stores.
    // row offsets are 32-bit within the batch row: T H d_v < 2^31
    // lane (l16, g) stores columns 32 p + 8 g .. + 7 of its row for each
    // pair p of column tiles (see the packing below)
    uint16_t *obase = a.o + (size_t)b * c.T * c.H * c.dv + col0 + 8 * g;
    float2 *sbase_st = a.stats ? a.stats + (size_t)b * c.T * c.H * a.NS + slice : nullptr;
    static_assert(C::CT % 2 == 0, "column tiles come in pairs");
    uint32_t pend_o[C::NQT][C::CT / 2][4];
    uint32_t pend_row[C::NQT];  // t H + h within the batch row
    float2 pend_stat[C::NQT];
#pragma unroll
    for (int u = 0; u < C::NQT; ++u) {
        pend_row[u] = (uint32_t)(i0 * BC + 16 * qt[u] + l16) * c.H + h;
        pend_stat[u] = make_float2(0.f, 0.f);
#pragma unroll
        for (int p = 0; p < C::CT / 2; ++p) pend_o[u][p][0] = pend_o[u][p][1] = pend_o[u][p][2] = pend_o[u][p][3] = 0u;
    }
    const bool stats_out = a.NS > 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM);
    const bool norm_here = a.NS == 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM);
    const int64_t rp0 = (!SO && (c.flags & MSR_FLAG_DECAY_ROWNORM)) ? row_pos0(c, b) : 0;
    auto flush_u = [&](int u) {
        uint16_t *dst = obase + pend_row[u] * (uint32_t)c.dv;
#pragma unroll
        for (int p = 0; p < C::CT / 2; ++p) {
            const u32x4 v4 = {pend_o[u][p][0], pend_o[u][p][1], pend_o[u][p][2], pend_o[u][p][3]};
            *reinterpret_cast<u32x4 *>(dst + p * 32) = v4;
        }
        if (stats_out && g == 0) sbase_st[pend_row[u] * (uint32_t)a.NS] = pend_stat[u];
    };
    auto flush = [&]() {
#pragma unroll
        for (int u = 0; u < C::NQT; ++u) flush_u(u);
    };

    if (!SO) write_st(St0);
    if (i1 > i0) {
        dma_v(i0, Vb0);
        if (!SO) load_q(i0, 0, C::NQ);
#pragma unroll
        for (int kb = 0; kb < C::R; ++kb) {
            load_kp_k(i0, kb);
            if (!SO) load_kp_p(i0, kb);
        }
    }

    f32x4 oacc[C::NQT][C::CT];
    auto chunk = [&](int ci, const char *Vc, char *Vn, const __bf16 *Sc, __bf16 *Sn) {
        const int t0 = ci * BC;
        // this chunk's V slice has landed once at most VWAIT newer operations
        // are outstanding (the prologue issued fewer: wait for all)
        if (ci == i0)
            wait_vm<0>();
        else if (SO)
            wait_vm<C::VWAIT_SO>();
        else
            wait_vm<C::VWAIT>();
        __syncthreads();
        if (SO) dma_v(ci + 1, Vn);
        if constexpr (!SO) {
            vmem_fence();
            prefetch(ci + 1);
            vmem_fence();
        }

        // ---- O^T = (S_old^T Q~^T) xi.  After the MFMAs of k-step ks, memory
        // operation ks of [previous outputs of tile 0..NQT-1, next V units]
        // is issued (the rest after the loop): stores first, then V.
        constexpr int NOPS = C::NQT + (C::V_FIRST ? C::NV : 0);
        auto op = [&](int i) {
            if (i < C::NQT) {
                flush_u(i);
            } else {
                dma_v_unit(ci + 1, i - C::NQT, Vn);
            }
        };
        if (!SO) {
            bf16x8 fr[2][C::CT];  // S_old^T fragments of k-steps ks (even/odd)
#pragma unroll
            for (int ct = 0; ct < C::CT; ++ct)
                fr[0][ct] = *reinterpret_cast<const bf16x8 *>(Sc + (ct * 16 + l16) * C::SP + 8 * g);
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                if (ks + 1 < C::KS) {
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct)
                        fr[(ks + 1) & 1][ct] =
                            *reinterpret_cast<const bf16x8 *>(Sc + (ct * 16 + l16) * C::SP + 32 * (ks + 1) + 8 * g);
                }
                vmem_fence();
#pragma unroll
                for (int u = 0; u < C::NQT; ++u)
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct)
                        oacc[u][ct] = mfma16(fr[ks & 1][ct], qr[u][ks],
                                             ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : oacc[u][ct]);
                vmem_fence();
                if (ks < NOPS) op(ks);
                vmem_fence();
            }
#pragma unroll
            for (int i = C::KS; i < NOPS; ++i) op(i);
            vmem_fence();
            // S_old = S^ gamma^(BC ph), times xi per query row (already in the
            // Q~ fragments when prep_kernel staged Q~ in LDS)
            if constexpr (!C::QSTAGE) {
                const float fx = exp2f((float)(BC * ph) * lg);
#pragma unroll
                for (int u = 0; u < C::NQT; ++u) {
                    const float x = xi[16 * qt[u] + l16] * fx;
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct) oacc[u][ct] = oacc[u][ct] * x;
                }
            }
        }
        if (!a.par) {  // a new run of the rescale period: S^ = gamma^BC S_old, phase 0
            const int j = ci % period;
            if (j == 0) {
                const float f = exp2f((float)(BC * (1 + ph)) * lg);
#pragma unroll
                for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                    for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = S[rt][ct] * f;
            }
            ph = j;
        }

        // ---- per 32-key block: state update and value product
#pragma unroll
        for (int kb = 0; kb < C::NB; ++kb) {
            if (!SO && !C::V_FIRST && kb == C::KBV) {
                vmem_fence();
                dma_v(ci + 1, Vn);
                vmem_fence();
            }
            // the block R ahead (in this chunk or the next) reuses this slot
            const int nb = kb + C::R;
            const int ci2 = ci + nb / C::NB, kb2 = nb % C::NB;
            // V of this block read transposed, keys in the order
            // {4g..4g+3, 16+4g..16+4g+3} of lane group g -- the order of the
            // P^T and (K~ zeta s)^T fragments.  When a wave's state tiles span
            // all value columns (CG == 1) one read serves both products.
            constexpr bool SHARE = !SO && C::CG == 1;
            constexpr int NVA = C::CT;
            s16x4 va[NVA][2];
            if constexpr (!SO) {
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) {
                    const int col = ct * 16 + 4 * (l16 & 3);
                    va[ct][0] = lds_tr(Vc + C::voff(32 * kb + 4 * g + (l16 >> 2), col));
                    va[ct][1] = lds_tr(Vc + C::voff(32 * kb + 16 + 4 * g + (l16 >> 2), col));
                }
            }
            {  // S += (K~ zeta s)^T V
                bf16x8 bv[C::CPW];
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct) {
                    if constexpr (SHARE) {
                        bv[ct] = cat(va[ct][0], va[ct][1]);
                    } else {
                        const int col = (cbase + ct) * 16 + 4 * (l16 & 3);
                        bv[ct] = cat(lds_tr(Vc + C::voff(32 * kb + 4 * g + (l16 >> 2), col)),
                                     lds_tr(Vc + C::voff(32 * kb + 16 + 4 * g + (l16 >> 2), col)));
                    }
                }
#pragma unroll
                for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                    for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = mfma16(kr[rt][kb % C::R], bv[ct], S[rt][ct]);
            }
            vmem_fence();
            load_kp_k(ci2, kb2);
            vmem_fence();
            if (!SO) {  // O^T += V^T P^T for the query tiles that reach this block
#pragma unroll
                for (int u = 0; u < C::NQT; ++u) {
                    if (!(32 * kb <= 16 * qt[u] + 15)) continue;
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct)
                        oacc[u][ct] = mfma16(cat(va[ct][0], va[ct][1]), pr[u][kb % C::R], oacc[u][ct]);
                }
            }
            vmem_fence();
            if (!SO) {
                load_kp_p(ci2, kb2);
                load_q(ci + 1, C::qpart0(kb), C::qpart0(kb + 1));
            }
            vmem_fence();
        }

        if (SO) return;
        // ---- GroupNorm over each row (lanes l16, l16+16, +32, +48 share a query)
#pragma unroll
        for (int u = 0; u < C::NQT; ++u) {
            const int jq = 16 * qt[u] + l16;
            pend_row[u] = (uint32_t)(t0 + jq) * c.H + h;
            if (c.flags & MSR_FLAG_DECAY_ROWNORM) {
                const float f = 1.f / decay_row_sum(rp0 + t0 + jq, lg);
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) oacc[u][ct] = oacc[u][ct] * f;
            }
            if (norm_here || stats_out) {
                float sum = 0.f;
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) sum += oacc[u][ct][0] + oacc[u][ct][1] + oacc[u][ct][2] + oacc[u][ct][3];
                const float mean = sum_lane_groups(sum) * (1.f / W);
                float m2 = 0.f;
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m2 += (oacc[u][ct][r] - mean) * (oacc[u][ct][r] - mean);
                m2 = sum_lane_groups(m2);
                pend_stat[u] = make_float2(mean, m2);
                if (norm_here) {
                    const float inv = 1.f / sqrtf(m2 * (1.f / W) + c.eps);
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                        for (int r = 0; r < 4; ++r) oacc[u][ct][r] = (oacc[u][ct][r] - mean) * inv;
                }
            }
            // Lane (l16, g) holds columns 16 ct + 4 g .. + 3 of row l16.
            // For each pair of column tiles, exchanging the upper half of
            // the first with the lower half of the second
            // (permlane32_swap), then the odd 16-lane rows of the first
            // result with the even rows of the second (permlane16_swap),
            // leaves columns 8 g .. 8 g + 7 of the pair in lane group g,
            // so each row of the pair leaves as one 64-byte piece.
#pragma unroll
            for (int p = 0; p < C::CT / 2; ++p)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const auto s32 =
                        __builtin_amdgcn_permlane32_swap(pack_bf16x2(oacc[u][2 * p][2 * i], oacc[u][2 * p][2 * i + 1]),
                                                         pack_bf16x2(oacc[u][2 * p + 1][2 * i], oacc[u][2 * p + 1][2 * i + 1]),
                                                         false, false);
                    const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
                    pend_o[u][p][i] = s16[0];
                    pend_o[u][p][2 + i] = s16[1];
                }
        }
        write_st(Sn);
    };
    for (int ci = i0; ci < i1; ci += 2) {
        chunk(ci, Vb0, Vb1, St0, St1);
        if (ci + 1 < i1) chunk(ci + 1, Vb1, Vb0, St1, St0);
    }
    if (!SO && i1 > i0) flush();

    if (SO && a.par) {  // the parallel form's outgoing state
        if (a.s_out) {
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = (rbase + rt) * 16 + 4 * g + r, col = (cbase + ct) * 16 + l16;
                        a.s_out[sbase + (size_t)row * c.dv + col] = S[rt][ct][r];
                    }
        }
    } else if (SO) {  // this segment's end state from a zero state
        const float f = exp2f((float)(BC * ph) * lg);
#pragma unroll
        for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = (rbase + rt) * 16 + 4 * g + r, col = (cbase + ct) * 16 + l16;
                    a.segE[ebase + ((size_t)seg * DK + row) * c.dv + col] = S[rt][ct][r] * f;
                }
    } else if (a.s_out && seg == a.nseg - 1) {
        const float f = exp2f((float)(BC * ph) * lg);
#pragma unroll
        for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = (rbase + rt) * 16 + 4 * g + r, col = (cbase + ct) * 16 + l16;
                    a.s_out[sbase + (size_t)row * c.dv + col] = S[rt][ct][r] * f;
                }
    }
    // the clamped loads of the last chunk may still be in flight
    __builtin_amdgcn_s_waitcnt(0);
}

// What a chunk kernel that did not wait for the slices' words needs at its
// end to normalise a (pair, segment)'s rows from them.
struct XgEnd {
    const unsigned long long *words;  // [pair][16-row tile][slice][16 rows], 8 bytes each
    uint16_t *o;
    unsigned *tick;  // the exchange's counters
    float eps;
    unsigned id;     // the call's id
    int ps;          // pair nseg + segment
    int NS, nseg, rows, T, H, dv;  // rows: of a segment
};

// The GroupNorm of pair's rows t0 .. t0 + e.rows - 1 from the slices' words
// (the slice's mean, then its M2 with the sign bit set), by one workgroup
// (threads tid of nt), a thread normalising 32 values of a row at a time.
// The row's mean is the mean of the slice means, its M2 the sum of the slice
// M2 plus W (slice mean - row mean)^2.
__device__ __forceinline__ void normalise_from_words(const XgEnd &e, int tid, int nt) {
    const int tpr = e.dv / 32;  // threads per row, 32 values each
    const int pair = e.ps / e.nseg, t0 = e.ps % e.nseg * e.rows;
    const int b = pair / e.H, h = pair % e.H;
    for (int gid = tid; gid < e.rows * tpr; gid += nt) {
        const int t = t0 + gid / tpr;
        const unsigned long long *wr = e.words + ((size_t)pair * e.T + (t & ~15)) * e.NS + (t & 15);
        float mean = 0.f;
        for (int sl = 0; sl < e.NS; ++sl) mean += __uint_as_float((uint32_t)wr[16 * sl]);
        mean /= (float)e.NS;
        float m2 = 0.f;
        for (int sl = 0; sl < e.NS; ++sl) {
            const float d = __uint_as_float((uint32_t)wr[16 * sl]) - mean;
            m2 += __uint_as_float((uint32_t)(wr[16 * sl] >> 32) & 0x7fffffffu) + (float)W * d * d;
        }
        const float inv = 1.f / sqrtf(m2 / (float)e.dv + e.eps);
        u32x4 *p = reinterpret_cast<u32x4 *>(e.o + (((size_t)b * e.T + t) * e.H + h) * e.dv) + gid % tpr;
        for (int i = 0; i < 4; ++i) {
            const u32x4 x = p[i * tpr];
            u32x4 y;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                y[k] = pack_bf16x2((__uint_as_float(x[k] << 16) - mean) * inv,
                                   (__uint_as_float(x[k] & 0xffff0000u) - mean) * inv);
            p[i * tpr] = y;
        }
    }
}

// Warp-specialised variant of the full pass (b <= 128): 8 waves, two per
// SIMD.  The four "O" waves (w < 4) run the inter-chunk product, the value
// product and GroupNorm with the fragments of chunk kernel wave w; the four
// "S" waves run the state update and the V loads with the state tiles of
// wave w - 4.  Both kinds meet at one barrier per chunk; the S waves write
// S_new^T for the next chunk's inter-chunk product into the other LDS
// buffer.  The kernel waits on memory most of the time (the fragments of a
// pair are read by all of its value slices, from L2, and V and O stream
// through HBM; at the 7B shape a call at B = 1 on half the CUs runs each
// workgroup twice as fast, so the shared L2-miss path, not the CU, sets the
// pace), so:
//   - each fragment load is issued right after the last use of its
//     registers, a chunk ahead of its next use (full scheduling barriers
//     keep the compiler from sinking the loads to the end of the chunk);
//   - V goes through registers (plain loads, stored to LDS at the end of the
//     chunk), so no direct-to-LDS load is outstanding when the compiler
//     waits for a fragment;
//   - P^T fragments of key blocks a query tile does not reach are not loaded;
//   - with 8 or more slices per pair, the S waves prefetch the pair's
//     fragment lines of the next chunk into L2, each slice its share.
//
// GroupNorm exchange (XG, 2 <= NS <= 8 slices per row).  The NS workgroups
// of a (pair, segment) run through the same chunks side by side, so instead
// of leaving slice partials to gn_finalize_kernel (a second pass over O),
// each O wave publishes the (mean, M2) of its rows' 64 columns at the end of
// a chunk, as one 8-byte word per row and slice written with a device-scope
// atomic store: the mean's bits, then M2's with the sign bit set, which marks
// the word as written (prep_kernel zeroes the words first; M2 >= 0).  A word
// is single-copy atomic, so no fence is needed.  The wave keeps the bf16
// outputs of chunk cj in an LDS ring, loads the NS words of their rows with
// device-scope atomic loads at the start of chunk cj + 2 (a whole chunk ahead
// of use, and a chunk after the slices wrote them), and at the end of chunk
// cj + 2, once every word is marked (reloading until then), combines them --
// mean of the slice means, M2 = sum of the slice M2 + 64 (mean_s - mean)^2 --
// and stores the normalised rows.  The words of a (pair, chunk) are laid out
// per 16-row tile as [slice][row], so that a slice's words of a tile are one
// cache line: the loads add few requests to a kernel bound by them.
// The wait cannot deadlock: workgroups take tickets from a counter in the
// order they start and the slices of a (pair, segment) hold consecutive
// tickets, so when any of them waits, all of the earliest waiting group have
// started, and that group never waits on a later one.  The slices run side by
// side only when the whole grid is resident at once, which the launch
// requires before it picks this mode, and only one call at a time may wait
// before its grid is all resident: its prep_kernel claims the device's
// exchange (g_xg_owner), which its last workgroup to start hands back.  A
// call that finds the exchange claimed by another runs the same code on
// neutral words (mean 0, scale 1: it never waits and stores its rows
// unnormalised), and the last of a (pair, segment)'s workgroups to finish
// normalises that segment's rows from the real words (one workgroup per
// segment, so slower; this only happens when calls overlap).  The wait is
// bounded (10 s per wave); rows whose words it never saw marked would be
// stored as NaN.
template <int DK, int BC, bool XG>
__global__ __launch_bounds__((2 * Cfg<DK, BC>::THREADS)) void chunk_ws_kernel(MsrConst c, ChunkArgs a) {
    using C = Cfg<DK, BC>;
    static_assert(C::NW == 4 && C::QSTAGE, "warp-specialised pass: 4 + 4 waves, Q~ fragments carry xi");
    __shared__ __attribute__((aligned(16))) char Vb0[C::VTILE], Vb1[C::VTILE];
    __shared__ __attribute__((aligned(16))) __bf16 St0[W * C::SP], St1[W * C::SP];  // S_old^T
    // exchange: each O wave's bf16 outputs of the last two chunks
    constexpr int RING = 2 * C::NW * C::NQT * (C::CT / 2) * 1024;
    static_assert(!XG || 2 * C::VTILE + 4 * W * C::SP + RING <= 163840, "LDS budget (exchange ring)");
    __shared__ __attribute__((aligned(16))) char Ob[XG ? RING : 16];

    const int tid = threadIdx.x, lane = tid & 63, w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool srole = w8 >= C::NW;
    const int w = srole ? w8 - C::NW : w8;
    const int l16 = lane & 15, g = lane >> 4;
    const int npairs = c.B * c.H;
    int pair, seg, slice;
    // exchange state that is read rarely, kept in LDS rather than in
    // registers across the chunk loop: the call's mode (1: wait for the
    // slices' words, 2: store rows raw) and what the kernel's end needs
    __shared__ unsigned xs_mode;
    __shared__ XgEnd xs_end;
    bool xlastq = false;  // (thread 0) the owner's last workgroup to start in its ticket queue
    unsigned xqc = 0u;    // (thread 0 of those) the queues counted, itself included (8: release the claim)
    {
        const int nps = npairs * a.nseg;
        int id = blockIdx.x;
        if constexpr (XG) {
            // tickets in start order, one queue per XCD-sized group of ids
            // when the (pair, segment) groups stay within one (see above),
            // and the call's mode in the ticket's top bit: 1 = wait for the
            // slices' words (this call owns the exchange), 2 = do not wait
            // (another call owns it).  The owner's last workgroup to start
            // hands the exchange back when it ends; with eight queues, the
            // last to start in each queue counts its queue, and the one that
            // counts the eighth hands it back (the count's reply is not
            // waited for at the start).
            __shared__ int ticket;
            if (tid == 0) {
                const int nq = nps % 8 == 0 ? 8 : 1;
                const int qu = nq == 8 ? (int)(blockIdx.x & 7) : 0;
                const unsigned tk = __hip_atomic_fetch_add(a.xtick + qu, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int t = (int)(tk & 0x7fffffffu);
                const unsigned md = tk >> 31 ? 2u : 1u;
                xlastq = md == 1u && t == (int)gridDim.x / nq - 1;
                ticket = nq == 8 ? 8 * t + qu : t;
                xs_mode = md;
            }
            __syncthreads();
            id = ticket;
            if (xlastq)
                xqc = nps % 8 == 0
                          ? __hip_atomic_fetch_add(a.xtick + 9, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u
                          : 8u;
        }
        int ps;
        if (nps % 8 == 0) {
            const int xcd = id & 7, j = id >> 3;
            ps = (j / a.NS) * 8 + xcd;
            slice = j % a.NS;
        } else {
            ps = id / a.NS;
            slice = id % a.NS;
        }
        pair = ps / a.nseg;
        seg = ps % a.nseg;
        if (XG && tid == 0)
            xs_end = XgEnd{reinterpret_cast<const unsigned long long *>(a.stats), a.o, a.xtick, c.eps, a.xid, ps,
                           a.NS, a.nseg, a.seglen * BC, c.T, c.H, c.dv};
    }
    const int i0 = seg * a.seglen, i1 = i0 + a.seglen;
    const int b = pair / c.H, h = pair % c.H;
    const int col0 = slice * W;
    const float lg = c.log2g[h];
    const int period = rescale_period(lg, BC);
    int ph = i0 == 0 ? 0 : (i0 - 1) % period;
    const int nch = c.T / BC;
    const size_t pc0 = (size_t)pair * nch;
    const uint16_t *qfb = a.qf + pc0 * (C::NKT * C::KS * FRAG);
    const uint16_t *kfb = a.kf + pc0 * (C::RT * C::NB * FRAG);
    const uint16_t *pfb = a.pf + pc0 * (C::NKT * C::NB * FRAG);
    const uint32_t loff = lane * 16;
    auto ldfrag = [&](const uint16_t *fb, size_t frag) {
        return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(fb + frag * FRAG) + loff);
    };
    const uint32_t rowV = (uint32_t)c.H * c.dv * 2;
    const char *vb = reinterpret_cast<const char *>(a.v + ((size_t)b * c.T * c.H + h) * c.dv + col0);

    if (srole) {
        // ------------------------------------------------------------ S waves
        const int rbase = (w / C::CG) * C::RPW, cbase = (w % C::CG) * C::CPW;
        // V slices go through registers (plain loads, written to LDS at the
        // end of the chunk): with no direct-to-LDS load outstanding, the
        // compiler's waits for the K~ fragments stay exact
        u32x4 vreg[C::NV];
        auto load_v = [&](int ci) {
            ci = ci < nch ? ci : nch - 1;
#pragma unroll
            for (int i = 0; i < C::NV; ++i) {
                const int unit = i * C::NW + w;
                const int byte = unit * 1024 + lane * 16;
                const int row = byte / C::VROW, phys = (byte % C::VROW) >> 4;
                vreg[i] = *reinterpret_cast<const u32x4 *>(vb + (uint32_t)(ci * BC + row) * rowV + (phys ^ C::swz_v(row)) * 16);
            }
        };
        auto store_v = [&](char *dst) {
#pragma unroll
            for (int i = 0; i < C::NV; ++i) *reinterpret_cast<u32x4 *>(dst + (i * C::NW + w) * 1024 + lane * 16) = vreg[i];
        };
        bf16x8 kr[C::RPW][C::R];
        auto load_kp_k = [&](int ci, int kb) {
            ci = ci < nch ? ci : nch - 1;
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt)
                kr[rt][kb % C::R] = ldfrag(kfb, (size_t)(ci * C::RT + rbase + rt) * C::NB + kb);
        };
        f32x4 S[C::RPW][C::CPW];
        const size_t sbase = (size_t)pair * DK * c.dv + col0;
        const size_t ebase = (size_t)pair * a.nseg * DK * c.dv + col0;
        // the incoming state: with segments, the copy the state-only pass made
        const float *sin_p = a.nseg > 1 ? a.segE + ebase + (size_t)(a.nseg - 1) * DK * c.dv
                                        : (a.s_in ? a.s_in + sbase : nullptr);
        {
            const float gseg = exp2f((float)(BC * a.seglen) * lg);
            const float f0 = exp2f(-(float)(BC * ph) * lg);
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = (rbase + rt) * 16 + 4 * g + r, col = (cbase + ct) * 16 + l16;
                        S[rt][ct][r] = sin_p ? sin_p[(size_t)row * c.dv + col] : 0.f;
                    }
            // earlier segments' end states
            fold_segments<64>(S, a.segE + ebase, (size_t)DK * c.dv, seg, gseg, [&](int rt, int ct, int r) {
                return (size_t)((rbase + rt) * 16 + 4 * g + r) * c.dv + (cbase + ct) * 16 + l16;
            });
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = S[rt][ct] * f0;
        }
        auto write_st = [&](__bf16 *St) {
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct) {
                    const int row = (rbase + rt) * 16 + 4 * g, col = (cbase + ct) * 16 + l16;
                    bf16x4 v4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v4[r] = static_cast<__bf16>(S[rt][ct][r]);
                    *reinterpret_cast<bf16x4 *>(St + col * C::SP + row) = v4;
                }
        };
        // L2 prefetch of the pair's fragments PD chunks ahead.  All NS slices
        // of a pair read every fragment line; without the prefetch the first
        // reads of a line miss L2, and loads return in order, so each miss
        // holds back the hits issued after it.  Slice s touches only its
        // 1/NS share of a chunk's lines, one dword per 128-byte line, so the
        // prefetch costs 1/NS extra requests per line: a gain at NS = 8 (the
        // 7B-shaped layer: 299 -> 281 us), a loss at NS = 4 (long sequence),
        // hence only from 8 slices.  The dword is kept live by an empty asm
        // a chunk later, so the compiler's in-order load counts stay exact.
        // One chunk ahead is far enough: at two or three, part of the
        // prefetched lines leave L2 before the slices read them and come in
        // twice (7B-shaped call: 621 MB fetched at one chunk ahead, 636 MB at
        // two, 893 MB at three; kernel time the same within the noise).
        constexpr int PD = 1;
        constexpr int QFB = C::NKT * C::KS * FRAG * 2, KFB = C::RT * C::NB * FRAG * 2, PFB = C::NKT * C::NB * FRAG * 2;
        constexpr int NL = (QFB + KFB + PFB) / 128;  // fragment lines per chunk
        const int lps = (NL + a.NS - 1) / a.NS;     // ... per slice
        const int pl = slice * lps + w * 64 + lane;  // this lane's line
        const bool pf_on = a.NS >= 8 && w * 64 + lane < lps && pl < NL;
        uint32_t pfv = 0u;
        auto prefetch = [&](int cj) {
            cj = cj < nch ? cj : nch - 1;
            const char *p = pl < QFB / 128   ? reinterpret_cast<const char *>(qfb) + (size_t)cj * QFB + pl * 128
                            : pl < (QFB + KFB) / 128
                                ? reinterpret_cast<const char *>(kfb) + (size_t)cj * KFB + (pl - QFB / 128) * 128
                                : reinterpret_cast<const char *>(pfb) + (size_t)cj * PFB + (pl - (QFB + KFB) / 128) * 128;
            asm volatile("" ::"v"(pfv));
            if (pf_on) pfv = *reinterpret_cast<const uint32_t *>(p);
        };
        write_st(St0);
        if (i1 > i0) {
            load_v(i0);
#pragma unroll
            for (int kb = 0; kb < C::R; ++kb) load_kp_k(i0, kb);
            store_v(Vb0);
        }
        auto chunk = [&](int ci, const char *Vc, char *Vn, __bf16 *Sn) {
            __syncthreads();
            load_v(ci + 1);
            sched_fence();
            prefetch(ci + PD);
            sched_fence();
            {
                const int j = ci % period;
                if (j == 0) {
                    const float f = exp2f((float)(BC * (1 + ph)) * lg);
#pragma unroll
                    for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                        for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = S[rt][ct] * f;
                }
                ph = j;
            }
#pragma unroll
            for (int kb = 0; kb < C::NB; ++kb) {
                const int nb = kb + C::R;
                const int ci2 = ci + nb / C::NB, kb2 = nb % C::NB;
                bf16x8 bv[C::CPW];
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct) {
                    const int col = (cbase + ct) * 16 + 4 * (l16 & 3);
                    bv[ct] = cat(lds_tr(Vc + C::voff(32 * kb + 4 * g + (l16 >> 2), col)),
                                 lds_tr(Vc + C::voff(32 * kb + 16 + 4 * g + (l16 >> 2), col)));
                }
#pragma unroll
                for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                    for (int ct = 0; ct < C::CPW; ++ct) S[rt][ct] = mfma16(kr[rt][kb % C::R], bv[ct], S[rt][ct]);
                // the next chunk's fragments of this block are loaded here,
                // a chunk ahead of their use (nothing moves across)
                sched_fence();
                load_kp_k(ci2, kb2);
                sched_fence();
            }
            store_v(Vn);
            write_st(Sn);
        };
        for (int ci = i0; ci < i1; ci += 2) {
            chunk(ci, Vb0, Vb1, St1);
            if (ci + 1 < i1) chunk(ci + 1, Vb1, Vb0, St0);
        }
        asm volatile("" ::"v"(pfv));
        if (a.s_out && seg == a.nseg - 1) {
            const float f = exp2f((float)(BC * ph) * lg);
#pragma unroll
            for (int rt = 0; rt < C::RPW; ++rt)
#pragma unroll
                for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = (rbase + rt) * 16 + 4 * g + r, col = (cbase + ct) * 16 + l16;
                        a.s_out[sbase + (size_t)row * c.dv + col] = S[rt][ct][r] * f;
                    }
        }
    } else {
        // ------------------------------------------------------------ O waves
        int qt[C::NQT];
#pragma unroll
        for (int i = 0; i < C::NQT; ++i) qt[i] = C::qtile(w, i);
        bf16x8 qr[C::NQT][C::KS];
        bf16x8 pr[C::NQT][C::R];
        auto load_q = [&](int ci, int f0, int f1) {
            ci = ci < nch ? ci : nch - 1;
#pragma unroll
            for (int f = 0; f < C::NQ; ++f)
                if (f >= f0 && f < f1)
                    qr[f / C::KS][f % C::KS] = ldfrag(qfb, (size_t)(ci * C::NKT + qt[f / C::KS]) * C::KS + f % C::KS);
        };
        // P^T fragments of the key blocks a query tile reaches (the others
        // are neither written nor used)
        auto load_kp_p = [&](int ci, int kb) {
            ci = ci < nch ? ci : nch - 1;
#pragma unroll
            for (int u = 0; u < C::NQT; ++u)
                if (32 * kb <= 16 * qt[u] + 15)
                    pr[u][kb % C::R] = ldfrag(pfb, (size_t)(ci * C::NKT + qt[u]) * C::NB + kb);
        };
        // lane (l16, g) stores columns 32 p + 8 g .. + 7 of its row for each
        // pair p of column tiles (see the packing below)
        uint16_t *obase = a.o + (size_t)b * c.T * c.H * c.dv + col0 + 8 * g;
        float2 *sbase_st = a.stats ? a.stats + (size_t)b * c.T * c.H * a.NS + slice : nullptr;
        static_assert(C::CT % 2 == 0, "column tiles come in pairs");
        uint32_t pend_o[C::NQT][C::CT / 2][4];
        uint32_t pend_row[C::NQT];
        float2 pend_stat[C::NQT];
#pragma unroll
        for (int u = 0; u < C::NQT; ++u) {
            pend_row[u] = (uint32_t)(i0 * BC + 16 * qt[u] + l16) * c.H + h;
            pend_stat[u] = make_float2(0.f, 0.f);
#pragma unroll
            for (int p = 0; p < C::CT / 2; ++p) pend_o[u][p][0] = pend_o[u][p][1] = pend_o[u][p][2] = pend_o[u][p][3] = 0u;
        }
        const bool stats_out = !XG && a.NS > 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM);
        const bool norm_here = !XG && a.NS == 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM);
        const int64_t rp0 = (c.flags & MSR_FLAG_DECAY_ROWNORM) ? row_pos0(c, b) : 0;
        auto flush_u = [&](int u) {
            uint16_t *dst = obase + pend_row[u] * (uint32_t)c.dv;
#pragma unroll
            for (int p = 0; p < C::CT / 2; ++p) {
                const u32x4 v4 = {pend_o[u][p][0], pend_o[u][p][1], pend_o[u][p][2], pend_o[u][p][3]};
                *reinterpret_cast<u32x4 *>(dst + p * 32) = v4;
            }
            if constexpr (!XG)
                if (stats_out && g == 0) sbase_st[pend_row[u] * (uint32_t)a.NS] = pend_stat[u];
        };
        // GroupNorm exchange: lane group g takes the words of slices g and
        // g + 4 of its row.  The bf16 outputs of chunk cj wait in LDS slot
        // cj & 1 until the end of chunk cj + 2; the words of chunk cj are
        // loaded at the start of chunk cj + 2, a whole chunk ahead of use.
        // Words of a (pair, chunk) are contiguous, per 16-row tile [slice][row]:
        // a slice's 16 words of a tile fill one 128-byte line, and a tile's
        // words for all slices NS lines.
        // A call that does not wait reads the neutral words instead (every
        // offset masked into them) and never finds a word unmarked.
        unsigned long long *const xw =
            XG ? reinterpret_cast<unsigned long long *>(a.stats) + (size_t)pair * nch * BC * a.NS : nullptr;
        const unsigned long long *xr = xw;
        uint32_t xmask = 0xffffffffu;
        if constexpr (XG) {
            if (__builtin_amdgcn_readfirstlane(xs_mode) != 1u) {
                xr = reinterpret_cast<const unsigned long long *>(a.xtick + xg_counter_words(npairs * a.nseg));
                xmask = NEUTRAL_WORDS - 1;
            }
        }
        unsigned long long xs[XG ? C::NQT : 1][2];
        auto xrow = [&](int cj, int u) { return (uint32_t)(cj * BC + 16 * qt[u] + l16) * c.H + h; };
        // word of (chunk cj, tile u, slice sl) for this lane's row
        auto xoff = [&](int cj, int u, int sl) { return (uint32_t)((cj * BC + 16 * qt[u]) * a.NS + sl * 16 + l16); };
        auto xword = [&](int cj, int u, int sl) { return xw + xoff(cj, u, sl); };
        const float rns = 1.f / (float)a.NS, rdv = 1.f / (float)c.dv;
        auto xload = [&](int cj, int u) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (g + 4 * j < a.NS)
                    xs[u][j] = __hip_atomic_load(xr + (xoff(cj, u, g + 4 * j) & xmask), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        };
        auto xmarked = [&](int u) {
            bool ok = true;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (g + 4 * j < a.NS) ok = ok && (xs[u][j] >> 63) != 0ull;
            return ok;
        };
        auto ring = [&](int cj, int u, int p) {
            return reinterpret_cast<u32x4 *>(Ob + ((((cj & 1) * C::NW + w) * C::NQT + u) * (C::CT / 2) + p) * 1024 +
                                             lane * 16);
        };
        // combine chunk cj's words, normalise its held-back outputs and store
        // them; the time a wave may spend waiting over the whole kernel is
        // bounded (10 s on the 100 MHz real-time counter)
        uint64_t xwaited = 0;
        auto xfinish = [&](int cj, int u) {
            if (!__all(xmarked(u)) && xwaited < 1000000000ull) {
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                do {
                    __builtin_amdgcn_s_sleep(2);
                    xload(cj, u);
                } while (!__all(xmarked(u)) && xwaited + (__builtin_amdgcn_s_memrealtime() - t0) < 1000000000ull);
                xwaited += __builtin_amdgcn_s_memrealtime() - t0;
            }
            float sm = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (g + 4 * j < a.NS) sm += __uint_as_float((uint32_t)xs[u][j]);
            const float mean = sum_lane_groups(sm) * rns;
            float m2 = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (g + 4 * j < a.NS) {
                    const float d = __uint_as_float((uint32_t)xs[u][j]) - mean;
                    m2 += __uint_as_float((uint32_t)(xs[u][j] >> 32) & 0x7fffffffu) + (float)W * d * d;
                }
            m2 = sum_lane_groups(m2);
            // (x - mean) / sqrt(var + eps) as one fma per value
            float inv = __builtin_amdgcn_rsqf(m2 * rdv + c.eps);
            if (!__all(xmarked(u))) inv = __builtin_nanf("");
            const float sh = -mean * inv;
            uint16_t *dst = obase + xrow(cj, u) * (uint32_t)c.dv;
#pragma unroll
            for (int p = 0; p < C::CT / 2; ++p) {
                u32x4 x = *ring(cj, u, p);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[e] = pack_bf16x2(__builtin_fmaf(__uint_as_float(x[e] << 16), inv, sh),
                                       __builtin_fmaf(__uint_as_float(x[e] & 0xffff0000u), inv, sh));
                *reinterpret_cast<u32x4 *>(dst + p * 32) = x;
            }
        };
        if (i1 > i0) {
            load_q(i0, 0, C::NQ);
#pragma unroll
            for (int kb = 0; kb < C::R; ++kb) load_kp_p(i0, kb);
        }
        f32x4 oacc[C::NQT][C::CT];
        auto chunk = [&](int ci, const char *Vc, const __bf16 *Sc) {
            const int t0 = ci * BC;
            __syncthreads();
            if constexpr (XG)
                if (ci - 2 >= i0) {
#pragma unroll
                    for (int u = 0; u < C::NQT; ++u) xload(ci - 2, u);
                }
            s16x4 va[2][C::CT][2];  // V^T of blocks kb (even/odd)
            auto read_va = [&](int kb, s16x4 (&d)[C::CT][2]) {
#pragma unroll
                for (int ct = 0; ct < C::CT; ++ct) {
                    const int col = ct * 16 + 4 * (l16 & 3);
                    d[ct][0] = lds_tr(Vc + C::voff(32 * kb + 4 * g + (l16 >> 2), col));
                    d[ct][1] = lds_tr(Vc + C::voff(32 * kb + 16 + 4 * g + (l16 >> 2), col));
                }
            };
            {
                constexpr int FD = C::KS >= 3 ? 2 : 1;  // S^T fragments read FD k-steps ahead
                bf16x8 fr[FD + 1][C::CT];
                auto read_fr = [&](int ks, bf16x8 (&d)[C::CT]) {
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct)
                        d[ct] = *reinterpret_cast<const bf16x8 *>(Sc + (ct * 16 + l16) * C::SP + 32 * ks + 8 * g);
                };
#pragma unroll
                for (int ks = 0; ks < FD; ++ks) read_fr(ks, fr[ks]);
                read_va(0, va[0]);
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    if (ks + FD < C::KS) read_fr(ks + FD, fr[(ks + FD) % (FD + 1)]);
                    vmem_fence();
#pragma unroll
                    for (int u = 0; u < C::NQT; ++u)
#pragma unroll
                        for (int ct = 0; ct < C::CT; ++ct)
                            oacc[u][ct] = mfma16(fr[ks % (FD + 1)][ct], qr[u][ks],
                                                 ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : oacc[u][ct]);
                    vmem_fence();
                    if (!XG && ks < C::NQT) flush_u(ks);
                    vmem_fence();
                }
                if constexpr (!XG) {
#pragma unroll
                    for (int i = C::KS; i < C::NQT; ++i) flush_u(i);
                }
                vmem_fence();
            }
#pragma unroll
            for (int kb = 0; kb < C::NB; ++kb) {
                const int nb = kb + C::R;
                const int ci2 = ci + nb / C::NB, kb2 = nb % C::NB;
                if (kb + 1 < C::NB) read_va(kb + 1, va[(kb + 1) & 1]);
#pragma unroll
                for (int u = 0; u < C::NQT; ++u) {
                    if (!(32 * kb <= 16 * qt[u] + 15)) continue;
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct)
                        oacc[u][ct] = mfma16(cat(va[kb & 1][ct][0], va[kb & 1][ct][1]), pr[u][kb % C::R], oacc[u][ct]);
                }
                sched_fence();
                load_kp_p(ci2, kb2);
                load_q(ci + 1, C::qpart0(kb), C::qpart0(kb + 1));
                sched_fence();
            }
#pragma unroll
            for (int u = 0; u < C::NQT; ++u) {
                if constexpr (XG)
                    if (ci - 2 >= i0) xfinish(ci - 2, u);
                const int jq = 16 * qt[u] + l16;
                pend_row[u] = (uint32_t)(t0 + jq) * c.H + h;
                if (c.flags & MSR_FLAG_DECAY_ROWNORM) {
                    const float f = 1.f / decay_row_sum(rp0 + t0 + jq, lg);
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct) oacc[u][ct] = oacc[u][ct] * f;
                }
                if constexpr (XG) {
                    float sum = 0.f;
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct) sum += oacc[u][ct][0] + oacc[u][ct][1] + oacc[u][ct][2] + oacc[u][ct][3];
                    const float mean = sum_lane_groups(sum) * (1.f / W);
                    float m2 = 0.f;
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                        for (int r = 0; r < 4; ++r) m2 += (oacc[u][ct][r] - mean) * (oacc[u][ct][r] - mean);
                    m2 = sum_lane_groups(m2);
                    if (g == 0)
                        __hip_atomic_store(xword(ci, u, slice),
                                           (unsigned long long)__float_as_uint(mean) |
                                               ((unsigned long long)(__float_as_uint(m2) | 0x80000000u) << 32),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else if (norm_here || stats_out) {
                    float sum = 0.f;
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct) sum += oacc[u][ct][0] + oacc[u][ct][1] + oacc[u][ct][2] + oacc[u][ct][3];
                    const float mean = sum_lane_groups(sum) * (1.f / W);
                    float m2 = 0.f;
#pragma unroll
                    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                        for (int r = 0; r < 4; ++r) m2 += (oacc[u][ct][r] - mean) * (oacc[u][ct][r] - mean);
                    m2 = sum_lane_groups(m2);
                    pend_stat[u] = make_float2(mean, m2);
                    if (norm_here) {
                        const float inv = 1.f / sqrtf(m2 * (1.f / W) + c.eps);
#pragma unroll
                        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
                            for (int r = 0; r < 4; ++r) oacc[u][ct][r] = (oacc[u][ct][r] - mean) * inv;
                    }
                }
                // the same lane swaps as in chunk_mfma_kernel: columns
                // 8 g .. + 7 of each pair of column tiles end in lane group g
#pragma unroll
                for (int p = 0; p < C::CT / 2; ++p)
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const auto s32 =
                            __builtin_amdgcn_permlane32_swap(pack_bf16x2(oacc[u][2 * p][2 * i], oacc[u][2 * p][2 * i + 1]),
                                                             pack_bf16x2(oacc[u][2 * p + 1][2 * i], oacc[u][2 * p + 1][2 * i + 1]),
                                                             false, false);
                        const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
                        pend_o[u][p][i] = s16[0];
                        pend_o[u][p][2 + i] = s16[1];
                    }
                if constexpr (XG) {
#pragma unroll
                    for (int p = 0; p < C::CT / 2; ++p)
                        *ring(ci, u, p) = u32x4{pend_o[u][p][0], pend_o[u][p][1], pend_o[u][p][2], pend_o[u][p][3]};
                }
            }
        };
        for (int ci = i0; ci < i1; ci += 2) {
            chunk(ci, Vb0, St0);
            if (ci + 1 < i1) chunk(ci + 1, Vb1, St1);
        }
        if (i1 > i0) {
            if constexpr (XG) {
                for (int cj = i1 - 2 >= i0 ? i1 - 2 : i0; cj < i1; ++cj) {
#pragma unroll
                    for (int u = 0; u < C::NQT; ++u) xload(cj, u);
#pragma unroll
                    for (int u = 0; u < C::NQT; ++u) xfinish(cj, u);
                }
            } else {
#pragma unroll
                for (int u = 0; u < C::NQT; ++u) flush_u(u);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (XG && xqc == 8u) {
        unsigned own = xs_end.id;
        __hip_atomic_compare_exchange_strong(&g_xg_owner, &own, 0u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
    }
    if (XG && xs_mode != 1u) {
        // After a call that did not wait, the last of the NS workgroups of a
        // (pair, segment) to finish normalises that segment's rows from the
        // slices' words (the others' rows and words are released before
        // their count, and acquired by it after the last count).
        __shared__ int last;
        __syncthreads();
        const XgEnd e = xs_end;
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // (a device-wide L2 write-back)
            last = __hip_atomic_fetch_add(e.tick + 16 + e.ps, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned)e.NS - 1;
        }
        __syncthreads();
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            normalise_from_words(e, tid, blockDim.x);
        }
    }
}

// Parallel form (jsqmd.com s4.1; aiqz.cc "parallel representation"):
//   O[n] = GN( sum_{m<=n} s gamma^(n-m) (q~_n . k~_m) v_m + gamma^(n+1) q~_n S_in )
// One workgroup of NWV waves per (pair, block of queries, value slice of PW
// columns: 256 when d_v allows, else 64); each wave owns NQW query tiles of
// 16, so a block holds 64, 128 or (eight waves) 256 queries.  The scores are
// formed once per slice, so the wider slice does them a quarter as often,
// and every wave of the workgroup shares the loads of a key block: the kernel
// is bound by the loads each CU keeps in flight, so more queries per load
// means more matrix work per request.  Per 32-key block up to the
// diagonal, the K~ fragments (prep_kernel, PAR) and the V slice stream into
// double-buffered LDS by direct loads; each wave forms P^T = K~ Q~^T with
// bf16 MFMA, applies s gamma^(n-m) and the causal mask in registers, and
// feeds P^T (two result tiles, keys in the order {4g..4g+3, 16+4g..}) as the
// B operand of O^T += V^T P^T, V^T read in that order with the transpose
// read.  The incoming-state term comes first, with S_in^T staged in LDS as
// bf16.  GroupNorm as in the chunk kernel.
struct ParArgs {
    const uint16_t *qf, *kq;  // Q~ and K~ fragments (prep_kernel<dk, 64, PAR>)
    const uint16_t *v;
    uint16_t *o;
    const float *s_in;
    float2 *stats;
    int NS;
};

template <int DK, int PW, int NQW, int NWV = 4>
__global__ __launch_bounds__(64 * NWV) void parallel_mfma_kernel(MsrConst c, ParArgs a) {
    using C = Cfg<DK, 64>;
    constexpr int KS = DK / 32;
    constexpr int CT = PW / 16;            // 16-column tiles of the slice
    constexpr int NT = NWV * NQW;          // query tiles per workgroup
    constexpr int QB = 16 * NT;            // queries per workgroup
    constexpr int KBYTES = 2 * KS * 1024;  // K~ fragments of one 32-key block
    constexpr int VBYTES = 32 * PW * 2;    // V slice of one 32-key block
    constexpr int NVL = VBYTES / 1024 / NWV;  // 1 KiB direct loads of it per wave
    static_assert(PW % 64 == 0 && NVL >= 1 && NVL * NWV * 1024 == VBYTES && (NQW == 1 || NQW == 2) &&
                      (NWV == 4 || NWV == 8),
                  "slice width, query tiles per wave, waves");
    // V rows (PW 2 bytes) with their 16-byte chunks XOR-swizzled by row so
    // that the transpose reads of a 16-lane group (4 rows x 32 bytes) spread
    // over the banks
    auto vswz = [](int r) { return PW == 64 ? (r >> 1) & 7 : ((r & 3) << 1) | ((r >> 2) & 1); };
    // K~ and V double buffers; before the first block the same LDS holds
    // S_in^T, 64 columns at a time (so that two workgroups fit on a CU)
    __shared__ __attribute__((aligned(16))) char L[2 * KBYTES + 2 * VBYTES];
    static_assert(W * C::SP * 2 <= 2 * KBYTES + 2 * VBYTES, "S_in^T staging fits the K~/V buffers");
    char *const Kb0 = L, *const Kb1 = L + KBYTES, *const Vb0 = L + 2 * KBYTES, *const Vb1 = L + 2 * KBYTES + VBYTES;
    __bf16 *const St = reinterpret_cast<__bf16 *>(L);

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int nqb = c.T / QB;
    // workgroup -> (pair, query block, slice).  Query block qb takes qb + 1
    // key-block units of work, so the workgroups are dispatched latest query
    // block first (the short ones fill the end); with pairs a multiple of 8,
    // the workgroups of one pair get ids equal mod 8 and run on one XCD,
    // whose L2 then serves its K~ and V blocks to all of them.
    int slice, qb, pair;
    {
        const int id = blockIdx.x, npairs = c.B * c.H;
        if (npairs % 8 == 0) {
            const int xcd = id & 7, j = id >> 3, pl = npairs / 8;
            slice = j % a.NS;
            const int pq = j / a.NS;
            pair = (pq % pl) * 8 + xcd;
            qb = nqb - 1 - pq / pl;
        } else {
            slice = id % a.NS;
            pair = (id / a.NS) % npairs;
            qb = nqb - 1 - id / a.NS / npairs;
        }
    }
    const int b = pair / c.H, h = pair % c.H;
    const int col0 = slice * PW;
    const float lg = c.log2g[h];
    // this wave's query tiles: NT qb + w, and with two per wave also
    // NT qb + NT - 1 - w (equal causal work across the waves)
    int tile[NQW], n[NQW];
#pragma unroll
    for (int i = 0; i < NQW; ++i) {
        tile[i] = i == 0 ? NT * qb + w : NT * qb + NT - 1 - w;
        n[i] = 16 * tile[i] + l16;  // this lane's query row (as MFMA column)
    }
    const uint32_t loff = lane * 16;
    // (Q~ and K~ fragments in prep_kernel's blocks of 64 queries)
    const uint16_t *qfb = a.qf + (size_t)pair * (c.T / 64) * (4 * KS * FRAG);
    const uint16_t *kqb = a.kq + (size_t)pair * (c.T / 64) * (4 * KS * FRAG);
    const uint32_t rowV = (uint32_t)c.H * c.dv * 2;
    const char *vb = reinterpret_cast<const char *>(a.v + ((size_t)b * c.T * c.H + h) * c.dv + col0);

    // key block kb: K~ fragments of key tiles 2 kb, 2 kb + 1 are 2 KS
    // consecutive fragments of the Q~-layout array; V rows 32 kb ..
    auto dma = [&](int kb, char *kd, char *vd) {
        const char *ks = reinterpret_cast<const char *>(kqb + (size_t)(2 * kb) * KS * FRAG);
        for (int u = w; u < 2 * KS; u += NWV) load_lds16(ks + u * 1024 + loff, kd + u * 1024);
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int unit = NWV * i + w, byte = unit * 1024 + lane * 16;
            const int row = byte / (PW * 2), phys = (byte % (PW * 2)) >> 4;
            load_lds16(vb + (uint32_t)(32 * kb + row) * rowV + (phys ^ vswz(row)) * 16, vd + unit * 1024);
        }
    };

    bf16x8 qr[NQW][KS];
#pragma unroll
    for (int i = 0; i < NQW; ++i)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qr[i][ks] = *reinterpret_cast<const bf16x8 *>(
                reinterpret_cast<const char *>(qfb + (size_t)(tile[i] * KS + ks) * FRAG) + loff);

    f32x4 oacc[NQW][CT];
#pragma unroll
    for (int i = 0; i < NQW; ++i)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) oacc[i][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.s_in) {  // (S_in^T Q~^T) gamma^(n+1), 64 value columns at a time
#pragma unroll
        for (int sc = 0; sc < PW / W; ++sc) {
            const float *sp = a.s_in + (size_t)pair * DK * c.dv + col0 + sc * W;
            if (sc > 0) __syncthreads();  // every wave is done with the previous columns
            for (int e = tid; e < DK * W; e += 64 * NWV) {
                const int row = e / W, col = e % W;
                St[col * C::SP + row] = static_cast<__bf16>(sp[(size_t)row * c.dv + col]);
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < W / 16; ++t) {
                    const bf16x8 A = *reinterpret_cast<const bf16x8 *>(St + (t * 16 + l16) * C::SP + 32 * ks + 8 * g);
#pragma unroll
                    for (int i = 0; i < NQW; ++i)
                        oacc[i][sc * (W / 16) + t] = mfma16(A, qr[i][ks], oacc[i][sc * (W / 16) + t]);
                }
        }
#pragma unroll
        for (int i = 0; i < NQW; ++i) {
            const float x = exp2f((float)(n[i] + 1) * lg);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) oacc[i][ct] = oacc[i][ct] * x;
        }
        __syncthreads();  // every wave is done with S_in^T before the loads overwrite it
    }

    // Decay of score (query n, key m = 32 kb + o), o = 16 v2 + 4 g + r the key
    // offset this lane holds:
    //   s gamma^(n - m) = [s gamma^(n - 32 kb - 31) gamma^(31 - 4 g)] gamma^(-(16 v2 + r)),
    // one exponential per tile and block times a lane factor, times one of
    // eight wave-uniform factors (gamma >= 0.9 on this path: every factor
    // stays below gamma^-31 < 27, and their product is gamma^(n - m) <= 1)
    const float dg = exp2f((float)(31 - 4 * g) * lg);
    float du[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        du[e] = __uint_as_float(__builtin_amdgcn_readfirstlane(
            __float_as_uint(exp2f(-(float)(16 * (e >> 2) + (e & 3)) * lg))));

    // V^T transpose-read addresses: lane rows rv and rv + 16, columns
    // 16 ct + 4 (l16 & 3); the 16-byte chunk 2 ct + b of the row is stored at
    // (2 ct + b) ^ sw = 2 (ct ^ (sw >> 1)) + (b ^ (sw & 1)), and sw >> 1 < 4 only
    // changes the low two bits of ct: four lane bases cover every ct, the rest
    // is an immediate offset
    const int rv = 4 * g + (l16 >> 2), sv = vswz(rv);  // (vswz(rv + 16) = vswz(rv))
    uint32_t vl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        vl[k] = rv * (PW * 2) + 32 * (k ^ (sv >> 1)) + 16 * (((l16 & 3) >> 1) ^ (sv & 1)) + 8 * (l16 & 1);

    const int nkb = (QB / 32) * (qb + 1);  // key blocks up to the workgroup's last query
    dma(0, Kb0, Vb0);
    auto block = [&](int kb, const char *Kc, const char *Vc, char *Kn, char *Vn) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kb + 1 < nkb) dma(kb + 1, Kn, Vn);
        // Skip the block when none of the wave's tiles reaches it.  A tile
        // that does not (the first of two, near the diagonal) is still
        // computed: its scores all fall under the causal mask, so it adds
        // zero, and the products stay one straight run of MFMAs -- guarding
        // each product by the tile turns every MFMA into a basic block of its
        // own, which the scheduler cannot overlap with the LDS reads.
        bool any = false;
#pragma unroll
        for (int i = 0; i < NQW; ++i) any = any || 32 * kb <= 16 * tile[i] + 15;
        if (!any) return;
        f32x4 acc[NQW][2];
#pragma unroll
        for (int i = 0; i < NQW; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int v2 = 0; v2 < 2; ++v2) {
                const bf16x8 A = *reinterpret_cast<const bf16x8 *>(Kc + (v2 * KS + ks) * 1024 + loff);
#pragma unroll
                for (int i = 0; i < NQW; ++i) acc[i][v2] = mfma16(A, qr[i][ks], acc[i][v2]);
            }
        bf16x8 pb[NQW];
#pragma unroll
        for (int i = 0; i < NQW; ++i) {
            const float base = c.scale * exp2f((float)(n[i] - 32 * kb - 31) * lg) * dg;
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = base * du[e];
            if (32 * kb + 31 <= 16 * tile[i]) {  // (uniform) every key before every query of the tile
#pragma unroll
                for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) pb[i][4 * v2 + r] = static_cast<__bf16>(acc[i][v2][r] * f[4 * v2 + r]);
            } else {
#pragma unroll
                for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 32 * kb + 16 * v2 + 4 * g + r;
                        pb[i][4 * v2 + r] = static_cast<__bf16>(m <= n[i] ? acc[i][v2][r] * f[4 * v2 + r] : 0.f);
                    }
            }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const char *va = Vc + vl[ct & 3] + 128 * (ct >> 2);
            const s16x4 v0 = lds_tr(va);
            const s16x4 v1 = lds_tr(va + 16 * PW * 2);
            const bf16x8 Vf = cat(v0, v1);
#pragma unroll
            for (int i = 0; i < NQW; ++i) oacc[i][ct] = mfma16(Vf, pb[i], oacc[i][ct]);
        }
    };
    for (int kb = 0; kb < nkb; kb += 2) {
        block(kb, Kb0, Vb0, Kb1, Vb1);
        if (kb + 1 < nkb) block(kb + 1, Kb1, Vb1, Kb0, Vb0);
    }

    // GroupNorm (in-wave when d_v == 64, else slice statistics) and store
    const bool stats_out = a.NS > 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM);
    const bool norm_here = a.NS == 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM);
#pragma unroll
    for (int i = 0; i < NQW; ++i) {
        const uint32_t rowi = (uint32_t)n[i] * c.H + h;  // token-head row within the batch row
        if (c.flags & MSR_FLAG_DECAY_ROWNORM) {
            const float f = 1.f / decay_row_sum(row_pos0(c, b) + n[i], lg);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) oacc[i][ct] = oacc[i][ct] * f;
        }
        if (norm_here || stats_out) {
            float sum = 0.f;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) sum += oacc[i][ct][0] + oacc[i][ct][1] + oacc[i][ct][2] + oacc[i][ct][3];
            const float mean = sum_lane_groups(sum) * (1.f / PW);
            float m2 = 0.f;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) m2 += (oacc[i][ct][r] - mean) * (oacc[i][ct][r] - mean);
            m2 = sum_lane_groups(m2);
            if (stats_out && g == 0)
                a.stats[((size_t)b * c.T * c.H + rowi) * a.NS + slice] = make_float2(mean, m2);
            if (norm_here) {
                const float inv = 1.f / sqrtf(m2 * (1.f / PW) + c.eps);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) oacc[i][ct][r] = (oacc[i][ct][r] - mean) * inv;
            }
        }
        uint16_t *dst = a.o + ((size_t)b * c.T * c.H + rowi) * c.dv + col0 + 4 * g;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const u32x2 v2 = {pack_bf16x2(oacc[i][ct][0], oacc[i][ct][1]), pack_bf16x2(oacc[i][ct][2], oacc[i][ct][3])};
            *reinterpret_cast<u32x2 *>(dst + ct * 16) = v2;
        }
    }
}

// GroupNorm of rows whose NS slices wrote (mean, M2) statistics over
// n = d_v / NS values each: the row's mean is the mean of the slice means and
// its M2 the sum of the slice M2 plus n (slice mean - row mean)^2 (the
// pairwise-update formula of Chan, Golub and LeVeque for equal counts).  A thread normalises 32
// values of one row in place (four 16-byte pieces, d_v / 32 threads per row)
// and combines that row's statistics (over a butterfly of lane exchanges
// among the row's threads when their count is a power of two); O is
// streamed with non-temporal loads and stores.
__global__ __launch_bounds__(256) void gn_finalize_kernel(MsrConst c, int NS, const float2 *__restrict__ stats,
                                                          uint16_t *__restrict__ o, size_t rows) {
    const int tpr = c.dv / 32;            // threads per row
    const float wn = (float)(c.dv / NS);  // values per slice
    const size_t gid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t row = gid / tpr;
    const int j = (int)(gid % tpr);
    if (row >= rows) return;
    u32x4 *p = reinterpret_cast<u32x4 *>(o + row * c.dv) + j;
    u32x4 u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = __builtin_nontemporal_load(p + i * tpr);
    const float2 *st = stats + row * NS;
    float mean = 0.f, m2 = 0.f;
    if ((tpr & (tpr - 1)) == 0 && NS <= tpr) {
        // the row's tpr threads are consecutive lanes of one wave (tpr is a
        // power of two <= 32): thread j takes slice j (if any) and the
        // partials combine pairwise over a butterfly of lane exchanges
        float n = 0.f;
        if (j < NS) {
            const float2 sj = st[j];
            n = wn;
            mean = sj.x;
            m2 = sj.y;
        }
        for (int off = 1; off < tpr; off <<= 1) {
            const float nb = __shfl_xor(n, off), mb = __shfl_xor(mean, off), m2b = __shfl_xor(m2, off);
            const float nn = n + nb;
            if (nn > 0.f) {
                const float d = mb - mean, fb = nb / nn;
                mean += d * fb;
                m2 += m2b + d * d * n * fb;
            }
            n = nn;
        }
    } else {
        float2 sv[MSR_MAX_DV / 32];
#pragma unroll
        for (int s = 0; s < MSR_MAX_DV / 32; ++s)
            if (s < NS) {
                sv[s] = st[s];
                mean += sv[s].x;
            }
        mean /= (float)NS;
#pragma unroll
        for (int s = 0; s < MSR_MAX_DV / 32; ++s)
            if (s < NS) {
                const float d = sv[s].x - mean;
                m2 += sv[s].y + wn * d * d;
            }
    }
    const float inv = 1.f / sqrtf(m2 / (float)c.dv + c.eps);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y[e] = pack_bf16x2((__uint_as_float(u[i][e] << 16) - mean) * inv,
                               (__uint_as_float(u[i][e] & 0xffff0000u) - mean) * inv);
        __builtin_nontemporal_store(y, p + i * tpr);
    }
}

// Workgroups of the persistent kernel KERN (threads per workgroup given)
// that the current device holds at once, at most nblk: its compute units
// times the workgroups one unit keeps resident (cached per device).
template <auto KERN>
unsigned fill_grid(int threads, size_t nblk) {
    static int resident[64];  // 0: not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int n = resident[dev];
    if (n == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, KERN, threads, 0) != hipSuccess || per <= 0) per = 1;
        n = cus * per;
        resident[dev] = n;
    }
    return (unsigned)(nblk < (size_t)n ? nblk : (size_t)n);
}

// Workgroups of the exchanging chunk_ws_kernel<dk, b> the current device
// holds at once (0 where that kernel does not exist).
template <int DK, int BC>
unsigned xg_resident_bc() {
    using C = Cfg<DK, BC>;
    if constexpr (C::NW == 4 && C::QSTAGE)
        return fill_grid<chunk_ws_kernel<DK, BC, true>>(2 * C::THREADS, (size_t)1 << 30);
    else
        return 0;
}
unsigned xg_resident(int dk, int bc) {
    switch (dk * 1000 + bc) {
    case 64064: return xg_resident_bc<64, 64>();
    case 64128: return xg_resident_bc<64, 128>();
    case 128064: return xg_resident_bc<128, 64>();
    case 128128: return xg_resident_bc<128, 128>();
    case 256064: return xg_resident_bc<256, 64>();
    case 256128: return xg_resident_bc<256, 128>();
    default: return 0;
    }
}

template <int DK, int BC, bool QPERM>
void launch_prep(const MsrConst &c, const ChunkArgs &a, const void *Q, const void *K, const void *Qlo,
                 const void *Klo, hipStream_t st) {
    using C = Cfg<DK, BC>;
    const size_t nblk = (size_t)c.B * c.H * (c.T / BC);
    if (Qlo && Klo) {
        constexpr auto pk = prep_kernel<DK, BC, false, true, QPERM>;
        const unsigned grid = C::PREP_PERSIST ? fill_grid<pk>(C::PREP_NT, nblk) : (unsigned)nblk;
        hipLaunchKernelGGL(pk, dim3(grid), dim3(C::PREP_NT), 0, st, c, static_cast<const uint16_t *>(Q),
                           static_cast<const uint16_t *>(K), const_cast<uint16_t *>(a.qf),
                           const_cast<uint16_t *>(a.kf), const_cast<uint16_t *>(a.pf), (uint16_t *)nullptr,
                           static_cast<const uint16_t *>(Qlo), static_cast<const uint16_t *>(Klo),
                           a.xtick ? reinterpret_cast<unsigned long long *>(a.stats) : nullptr, a.NS, a.xtick, a.xid,
                           c.B * c.H * a.nseg);
    } else {
        constexpr auto pk = prep_kernel<DK, BC, false, false, QPERM>;
        const unsigned grid = C::PREP_PERSIST ? fill_grid<pk>(C::PREP_NT, nblk) : (unsigned)nblk;
        hipLaunchKernelGGL(pk, dim3(grid), dim3(C::PREP_NT), 0, st, c, static_cast<const uint16_t *>(Q),
                           static_cast<const uint16_t *>(K), const_cast<uint16_t *>(a.qf),
                           const_cast<uint16_t *>(a.kf), const_cast<uint16_t *>(a.pf), (uint16_t *)nullptr,
                           (const uint16_t *)nullptr, (const uint16_t *)nullptr,
                           a.xtick ? reinterpret_cast<unsigned long long *>(a.stats) : nullptr, a.NS, a.xtick, a.xid,
                           c.B * c.H * a.nseg);
    }
}

template <int DK, int BC>
hipError_t launch_chunk(const MsrConst &c, const ChunkArgs &a, bool wide, const void *Q, const void *K,
                        const void *Qlo, const void *Klo, hipStream_t st) {
    using C = Cfg<DK, BC>;
    hipError_t e = hipSuccess;
    if constexpr (C::QSTAGE && BC <= 128 && DK >= 128) {
        if (wide) {  // 256-column slices (k_chunk_wide.hip)
            launch_prep<DK, BC, true>(c, a, Q, K, Qlo, Klo, st);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (a.nseg > 1 && (e = launch_chunk_wide(c, a, BC, true, st)) != hipSuccess) return e;
            main_kernel_begin(st);
            e = launch_chunk_wide(c, a, BC, false, st);
            main_kernel_end(st);
            return e;
        }
    }
    if (wide) return hipErrorNotSupported;
    launch_prep<DK, BC, false>(c, a, Q, K, Qlo, Klo, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int grid = c.B * c.H * a.nseg * a.NS;
    if (a.nseg > 1) {  // end states of segments 0 .. nseg-2
        auto sk = chunk_mfma_kernel<DK, BC, true>;
        hipLaunchKernelGGL(sk, dim3(grid), dim3(C::THREADS), 0, st, c, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if constexpr (C::NW == 4 && C::QSTAGE) {
        if (a.xtick)
            launch_main(chunk_ws_kernel<DK, BC, true>, dim3(grid), dim3(2 * C::THREADS), st, c, a);
        else
            launch_main(chunk_ws_kernel<DK, BC, false>, dim3(grid), dim3(2 * C::THREADS), st, c, a);
    } else {
        launch_main(chunk_mfma_kernel<DK, BC, false>, dim3(grid), dim3(C::THREADS), st, c, a);
    }
    return hipGetLastError();
}

template <int DK>
hipError_t dispatch_bc(const MsrConst &c, const ChunkArgs &a, bool wide, int chunk, const void *Q, const void *K,
                       const void *Qlo, const void *Klo, hipStream_t st) {
    switch (chunk) {
    case 64: return launch_chunk<DK, 64>(c, a, wide, Q, K, Qlo, Klo, st);
    case 128: return launch_chunk<DK, 128>(c, a, wide, Q, K, Qlo, Klo, st);
    case 256: return launch_chunk<DK, 256>(c, a, wide, Q, K, Qlo, Klo, st);
    default: return hipErrorNotSupported;
    }
}

struct MfmaPlan {
    size_t qf = 0, kf = 0, pf = 0, stats = 0, segE = 0, tick = 0, total = 0;
    int nseg = 1;
    int NS = 1;          // GroupNorm partials per row
    bool wide = false;   // 256-column slices (k_chunk_wide.hip)
    bool fused = false;  // the fused kernel (k_chunk_fused.hip): no fragments
    bool xg = false;     // the GroupNorm exchange may be used (chunk_ws_kernel; space for its counters)
};

// Segments per pair: doubled while the workgroups (pairs x value slices x
// segments) stay within one per CU and every segment keeps >= 2 chunks.
int choose_nseg(const msr_problem *p, int chunk, int slice_cols) {
    const int nch = p->T / chunk;
    const long units = (long)p->B * p->H * (p->dv / slice_cols);
    int g = 1;
    while (units * g * 2 <= 256 && nch % (g * 2) == 0 && nch / (g * 2) >= 2) g *= 2;
    return g;
}

// workspace: [QF][KF][PF][slice statistics][segment states]; the fused
// kernel (split = false: the caller's Q and K, no low parts) needs only
// [slice statistics][segment states]
MfmaPlan mfma_plan(const msr_problem *p, int chunk, bool split = false) {
    MfmaPlan m;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t tokens = (size_t)p->B * p->T * p->H;  // token-heads
    if (!split && (p->flags & MSR_FLAG_FUSED) && chunk_fused_supported(p->dk, p->dv, chunk) &&
        !(p->flags & (kFlagNoWide | MSR_FLAG_DECAY_ROWNORM))) {
        m.fused = true;
        m.NS = p->dv / 256;
        m.stats = 0;  // partials of 32 columns when the rows span several slices
        m.segE = m.NS > 1 ? up(tokens * (p->dv / 32) * sizeof(float2)) : 0;
        m.nseg = choose_nseg(p, chunk, 256);
        m.total = m.segE + (m.nseg > 1 ? up((size_t)p->B * p->H * m.nseg * p->dk * p->dv * sizeof(float)) : 0);
        return m;
    }
    m.qf = 0;
    m.kf = m.qf + up(tokens * p->dk * 2);
    m.pf = m.kf + up(tokens * p->dk * 2);
    // (b/16) x (b/32) fragments of 1 KiB per chunk: b * 2 bytes per token-head
    m.stats = m.pf + up(tokens * chunk * 2);
    // The wide-slice kernel when it needs no segments (one workgroup per
    // (pair, 256 columns) already fills the GPU: the decode prefill at
    // B = 64, 4.0 against 4.7 ms), and at b = 64 also when the 64-column
    // kernels would need segments too (the long sequence: 1.02 against
    // 1.04 ms).  Where the 64-column kernels fill the GPU without segments
    // and the wide one would not, they win: at the 7B-shaped layer 0.37
    // against 0.49 ms per call at b = 64, and at b = 128 the wide kernel's
    // faster full pass (253 against 303 us) does not pay for its 89 us
    // segment pass.
    const bool wide_ok = chunk_wide_supported(p->dk, p->dv, chunk) && !(p->flags & kFlagNoWide);
    m.wide = wide_ok && (choose_nseg(p, chunk, 256) == 1 || (chunk == 64 && choose_nseg(p, chunk, W) > 1));
    m.NS = p->dv / (m.wide ? 32 : W);  // GroupNorm partials per row
    // the warp-specialised kernel (b <= 128) normalises the rows itself when
    // they span 2 to 8 of its slices, exchanging slice statistics
    m.xg = !m.wide && chunk <= 128 && m.NS >= 2 && m.NS <= 8 && !(p->flags & MSR_FLAG_NO_GROUPNORM);
    m.segE = m.stats + (m.NS > 1 ? up(tokens * m.NS * sizeof(float2)) : 0);
    m.nseg = choose_nseg(p, chunk, m.wide ? 256 : W);
    m.tick = m.segE + (m.nseg > 1 ? up((size_t)p->B * p->H * m.nseg * p->dk * p->dv * sizeof(float)) : 0);
    m.total = m.tick + (m.xg ? xg_counter_words(p->B * p->H * m.nseg) * sizeof(unsigned) +
                                   NEUTRAL_WORDS * sizeof(unsigned long long)
                             : 0);
    return m;
}

// parallel form workspace: [QF][KQ][KF][slice statistics], blocks of 64
struct ParPlan {
    size_t qf = 0, kq = 0, kf = 0, stats = 0, total = 0;
};
ParPlan par_plan(const msr_problem *p) {
    ParPlan m;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t tokens = (size_t)p->B * p->T * p->H;
    const size_t frag = up(tokens * p->dk * 2);
    m.kq = frag;
    m.kf = 2 * frag;
    m.stats = 3 * frag;
    const int NS = p->dv / W;
    m.total = m.stats + (NS > 1 ? up(tokens * NS * sizeof(float2)) : 0);
    return m;
}

template <int DK>
hipError_t launch_parallel(const MsrConst &c, const msr_problem *p, const void *Q, const void *K, const void *V,
                           void *O, const float *s_in, float *s_out, void *ws, hipStream_t st) {
    const ParPlan m = par_plan(p);
    char *wsb = static_cast<char *>(ws);
    const int npairs = c.B * c.H, nqb = c.T / 64, NS = c.dv / W;
    const int PW = c.dv % 256 == 0 ? 256 : W;  // value columns per output workgroup
    const int NSO = c.dv / PW;                  // output slices (and GroupNorm partials) per row
    uint16_t *qf = reinterpret_cast<uint16_t *>(wsb + m.qf), *kq = reinterpret_cast<uint16_t *>(wsb + m.kq);
    uint16_t *kf = reinterpret_cast<uint16_t *>(wsb + m.kf);
    float2 *stats = NSO > 1 ? reinterpret_cast<float2 *>(wsb + m.stats) : nullptr;
    constexpr auto pk = prep_kernel<DK, 64, true>;
    const size_t pblk = (size_t)npairs * nqb;
    const unsigned pgrid = Cfg<DK, 64>::PREP_PERSIST ? fill_grid<pk>(Cfg<DK, 64>::PREP_NT, pblk) : (unsigned)pblk;
    hipLaunchKernelGGL(pk, dim3(pgrid), dim3(Cfg<DK, 64>::PREP_NT), 0, st, c, static_cast<const uint16_t *>(Q),
                       static_cast<const uint16_t *>(K), qf, kf, (uint16_t *)nullptr, kq, (const uint16_t *)nullptr,
                       (const uint16_t *)nullptr, (unsigned long long *)nullptr, 0, (unsigned *)nullptr, 0u, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ParArgs pa{qf, kq, static_cast<const uint16_t *>(V), static_cast<uint16_t *>(O), s_in, stats, NSO};
    // two query tiles per wave (128 queries per workgroup) when T allows: each
    // K~ and V fragment read from LDS then serves two MFMAs; with 256-column
    // slices and T a multiple of 256, eight waves (256 queries) share each
    // block's K~ and V loads
    const int nq2 = c.T % 128 == 0 ? 2 : 1;
    if (PW == 256 && c.T % 256 == 0) {
        launch_main(parallel_mfma_kernel<DK, 256, 2, 8>, dim3(npairs * (c.T / 256) * NSO), dim3(512), st, c, pa);
    } else {
        auto ok = PW == 256 ? (nq2 == 2 ? parallel_mfma_kernel<DK, 256, 2> : parallel_mfma_kernel<DK, 256, 1>)
                            : (nq2 == 2 ? parallel_mfma_kernel<DK, 64, 2> : parallel_mfma_kernel<DK, 64, 1>);
        launch_main(ok, dim3(npairs * (c.T / (64 * nq2)) * NSO), dim3(256), st, c, pa);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // outgoing state after the outputs, which read s_in (s_out may alias it)
    if (s_out) {
        ChunkArgs a{};
        a.qf = qf;
        a.kf = kf;
        a.pf = nullptr;
        a.v = static_cast<const uint16_t *>(V);
        a.o = static_cast<uint16_t *>(O);
        a.s_in = s_in;
        a.s_out = s_out;
        a.stats = nullptr;
        a.NS = NS;
        a.NW2 = NS;
        a.nseg = 1;
        a.seglen = nqb;
        a.segE = nullptr;
        a.par = 1;
        auto sk = chunk_mfma_kernel<DK, 64, true>;
        hipLaunchKernelGGL(sk, dim3(npairs * NS), dim3(Cfg<DK, 64>::THREADS), 0, st, c, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (NSO > 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM)) {
        const size_t rows = (size_t)p->B * p->T * p->H;
        const size_t blocks = (rows * (p->dv / 32) + 255) / 256;
        hipLaunchKernelGGL(gn_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, NSO, stats,
                           static_cast<uint16_t *>(O), rows);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

bool mfma_supported(const msr_problem *p, int form, int chunk) {
    if (p->dtype != MSR_BF16) return false;
    if (p->dk != 64 && p->dk != 128 && p->dk != 256) return false;
    if (p->dv % W != 0) return false;
    if (form == MSR_FORM_PARALLEL) {
        if (p->T < 64 || p->T % 64 != 0) return false;
    } else if (form == MSR_FORM_CHUNKWISE) {
        if (chunk != 64 && chunk != 128 && chunk != 256) return false;
        if (chunk > p->T || p->T % chunk != 0) return false;
    } else {
        return false;
    }
    // per-thread byte offsets within one batch row are 32-bit
    if ((uint64_t)p->T * p->H * (p->dk > p->dv ? p->dk : p->dv) * 2 >= (1ull << 32)) return false;
    return true;
}

size_t mfma_workspace_bytes(const msr_problem *p, int form, int chunk, bool split) {
    if (!mfma_supported(p, form, chunk)) return 0;
    return form == MSR_FORM_PARALLEL ? par_plan(p).total : mfma_plan(p, chunk, split).total;
}

hipError_t mfma_chunkwise(const MsrConst &c, const msr_problem *p, int chunk, const void *Q,
                          const void *K, const void *V, void *O, const float *s_in, float *s_out,
                          void *ws, hipStream_t st, const void *Qlo, const void *Klo) {
    const MfmaPlan m = mfma_plan(p, chunk, Qlo != nullptr);
    char *wsb = static_cast<char *>(ws);
    if (m.fused) {
        FusedArgs f{};
        f.q = static_cast<const uint16_t *>(Q);
        f.k = static_cast<const uint16_t *>(K);
        f.v = static_cast<const uint16_t *>(V);
        f.o = static_cast<uint16_t *>(O);
        f.s_in = s_in;
        f.s_out = s_out;
        f.stats = m.NS > 1 ? reinterpret_cast<float2 *>(wsb + m.stats) : nullptr;
        f.NS = m.NS;
        f.NW2 = m.NS;
        f.NP = p->dv / 32;
        f.nseg = m.nseg;
        f.seglen = p->T / chunk / m.nseg;
        f.segE = m.nseg > 1 ? reinterpret_cast<float *>(wsb + m.segE) : nullptr;
        hipError_t e = hipSuccess;
        if (m.nseg > 1 && (e = launch_chunk_fused(c, f, chunk, true, st)) != hipSuccess) return e;
        main_kernel_begin(st);
        e = launch_chunk_fused(c, f, chunk, false, st);
        main_kernel_end(st);
        if (e != hipSuccess) return e;
        if (m.NS > 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM)) {
            const size_t rows = (size_t)p->B * p->T * p->H;
            const size_t blocks = (rows * (p->dv / 32) + 255) / 256;
            hipLaunchKernelGGL(gn_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, f.NP, f.stats, f.o,
                               rows);
            e = hipGetLastError();
        }
        return e;
    }
    ChunkArgs a{};  // every field starts at zero (par = 0: chunkwise form)
    a.qf = reinterpret_cast<const uint16_t *>(wsb + m.qf);
    a.kf = reinterpret_cast<const uint16_t *>(wsb + m.kf);
    a.pf = reinterpret_cast<const uint16_t *>(wsb + m.pf);
    a.v = static_cast<const uint16_t *>(V);
    a.o = static_cast<uint16_t *>(O);
    a.s_in = s_in;
    a.s_out = s_out;
    a.NS = m.NS;
    a.NW2 = m.wide ? p->dv / 256 : a.NS;
    a.stats = a.NS > 1 ? reinterpret_cast<float2 *>(wsb + m.stats) : nullptr;
    a.nseg = m.nseg;
    a.seglen = p->T / chunk / m.nseg;
    a.segE = m.nseg > 1 ? reinterpret_cast<float *>(wsb + m.segE) : nullptr;
    // the exchange needs every slice of a (pair, segment) running at once:
    // the whole grid resident together (else the separate GroupNorm pass)
    const int xmode = exchange_mode();
    const bool xg = m.xg && xmode != MSR_EXCHANGE_OFF &&
                    (size_t)p->B * p->H * m.nseg * m.NS <= xg_resident(p->dk, chunk);
    a.xtick = xg ? reinterpret_cast<unsigned *>(wsb + m.tick) : nullptr;
    if (xg && xmode == MSR_EXCHANGE_AUTO) {  // a nonzero id per call claims the exchange (0: never waits)
        static std::atomic<unsigned> calls{0};
        unsigned id = ++calls;
        while (id == 0) id = ++calls;
        a.xid = id;
    }

    hipError_t e = hipSuccess;
    switch (p->dk) {
    case 64: e = dispatch_bc<64>(c, a, m.wide, chunk, Q, K, Qlo, Klo, st); break;
    case 128: e = dispatch_bc<128>(c, a, m.wide, chunk, Q, K, Qlo, Klo, st); break;
    case 256: e = dispatch_bc<256>(c, a, m.wide, chunk, Q, K, Qlo, Klo, st); break;
    default: e = hipErrorNotSupported;
    }
    if (e != hipSuccess) return e;
    if (a.NS > 1 && !xg && !(c.flags & MSR_FLAG_NO_GROUPNORM)) {
        const size_t rows = (size_t)p->B * p->T * p->H;
        const size_t blocks = (rows * (p->dv / 32) + 255) / 256;
        hipLaunchKernelGGL(gn_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, a.NS,
                           a.stats, a.o, rows);
        e = hipGetLastError();
    }
    return e;
}

hipError_t mfma_parallel(const MsrConst &c, const msr_problem *p, const void *Q, const void *K, const void *V,
                         void *O, const float *s_in, float *s_out, void *ws, hipStream_t st) {
    switch (p->dk) {
    case 64: return launch_parallel<64>(c, p, Q, K, V, O, s_in, s_out, ws, st);
    case 128: return launch_parallel<128>(c, p, Q, K, V, O, s_in, s_out, ws, st);
    case 256: return launch_parallel<256>(c, p, Q, K, V, O, s_in, s_out, ws, st);
    default: return hipErrorNotSupported;
    }
}
