// k_chunk_wide.hip -- wide-slice kernel of the chunkwise form (bf16 MFMA).
//
// The recurrence of chunk_mfma_kernel (jsqmd.com "From RoPE to Retention"
// s4.3; aiqz.cc RetNet tutorial, "chunkwise recurrence"):
//   O_i = GN( (Q~_i K~_i^T (.) D) V_i + (Q~_i S_{i-1}) (.) xi )
//   S_i = gamma^b S_{i-1} + K~_i^T (V_i (.) zeta)
// over the fragments prep_kernel writes (QF in its QPERM order, KF, PF), but a
// workgroup owns 256 value columns instead of 64.  Every value slice needs
// all of its chunk's QF, KF and PF fragments; with 64-column slices the chunk
// kernels fetch them from L2 once per 64 columns.  Here one fetch into LDS
// serves 256 columns.
//
// Workgroup: 8 waves, two per SIMD, owning (pair, 256 value columns, segment
// of chunks).  Wave w owns columns 32 w .. 32 w + 31 of the slice and keeps
// in MFMA accumulators its fp32 state S^[d_k][32] (RT x 2 tiles of 16x16)
// and the O^T[32][b/2] of half of the chunk's queries (2 x NKT/2 tiles).
// Per chunk, each wave takes the query halves in turn:
//   - O^T = S^T Q~^T (.) xi for the half.  The A operand is the wave's own
//     state, rounded to bf16 in registers: the 16x16 tiles of rows
//     32 ks .. 32 ks + 15 and 32 ks + 16 .. leave rows {4g..4g+3,
//     16+4g..16+4g+3} of the step in lane group g, which is the k order of
//     the QPERM fragments (a contraction index may be permuted in both
//     operands alike).  B = QF from LDS.
//   - O^T += V^T P^T over the key blocks the half reaches (V^T fragments by
//     the LDS transpose read, B = PF from LDS);
//   - GroupNorm partials (mean, M2) of each output row over its 32 columns
//     (gn_finalize_kernel combines them), O stored as bf16;
// and with the second half's value product, per 32-key block,
// S^ += (K~ zeta s)^T V (A = KF from LDS), after both inter-chunk products
// have read the old state.  S^ is the state up to the power of gamma
// described at rescale_period.
//
// Staging.  Per chunk the fragments arrive in NU units: QF of the first
// query half; V and P^T of the key blocks the first half reaches; QF of the
// second half; then per key block its KF fragments, the second half's P^T
// and the block's V rows.  A ring of NSLOT LDS slots is filled by direct
// buffer->LDS loads D = NSLOT - 1 units ahead, the waves sharing each unit's
// 1 KiB blocks.  At the start of a unit a wave waits for its own
// loads of it (a fixed vmcnt: every wave issues the same memory operations
// in the same order each chunk), then a barrier tells that all waves' loads
// have landed and that all waves are done with the slot the next loads
// overwrite, then it issues the unit D ahead and computes.

// Segments.  A workgroup per (pair, slice) alone would leave most CUs idle,
// so each pair's chunks are split into nseg segments.  The state-only
// instantiation (SO) computes the end state E_g of segments 0 .. nseg-2 from
// a zero state (the KF and V units only) and copies s_in aside; the full
// pass starts segment g from S_in(g) = gamma^(b seglen) S_in(g-1) + E_(g-1),
// S_in(0) = s_in (the chunkwise recurrence regrouped by segments).  Because
// the full pass then reads the incoming state only from the workspace, the
// outgoing state may overwrite it whatever order the workgroups run in.
#include <utility>

#include "msr_chunk.hpp"
#include "msr_device.hpp"

namespace {

using namespace msr;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NWV = 8;           // waves per workgroup
constexpr int WC = 32;           // value columns per wave
constexpr int WS = NWV * WC;     // value columns per workgroup
constexpr int CT = WC / 16;      // 16-column tiles per wave
constexpr int FB = 1024;         // bytes per operand fragment
constexpr int FE = 512;          // bf16 elements per operand fragment
constexpr int LDS_BYTES = 163840;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_addr(const char *p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char *)(p));
}

// Four LDS transpose reads (ds_read_b64_tr_b16: within each 16-lane group,
// lane j points at 4 consecutive bf16 of row r0 + j/4, columns c0 + 4 (j%4)
// ..; lane i then receives column c0 + i of rows r0 .. r0 + 3), complete
// when this returns: the wait for them is in the same asm block.  Written
// as asm because the compiler, which cannot tell that these reads do not
// touch LDS being filled by outstanding direct loads, would otherwise wait
// for all of them.
__device__ __forceinline__ void lds_tr4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, s16x4 &r0, s16x4 &r1,
                                        s16x4 &r2, s16x4 &r3) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}

__device__ __forceinline__ bf16x8 cat(s16x4 a, s16x4 b) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2 y = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, y);
}

// x[l] + x[l ^ 16] + x[l ^ 32] + x[l ^ 48] in every lane (gfx950 lane swaps)
__device__ __forceinline__ float sum_lane_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Buffer resource over nbytes from base (raw dword access; reads past the end
// return zeros)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane l reads at
// voff + soff and its bytes land at lds + 16 l (soff and lds are uniform)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, (int)voff,
                                             (int)soff, 0, 0);
}

// s_waitcnt with vmcnt = n and the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS: this wave's LDS reads are complete and no memory
// access moves across it.  Global loads stay in flight (a __syncthreads would
// wait for them).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int N, class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// XOR swizzle of the 16-byte chunks of a V row in LDS: the transpose reads of
// a 16-lane group (4 rows x 32 bytes) then touch 8 different bank groups
__host__ __device__ constexpr int vswz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int voff(int r, int col) {
    return r * (WS * 2) + ((((col >> 3) ^ vswz(r))) << 4) + (col & 7) * 2;
}

constexpr int max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

// Keeps the scheduler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int DK, int BC, bool SO>
struct WCfg {
    static constexpr int NKT = BC / 16;           // 16-token tiles per chunk
    static constexpr int NH = NKT / 2;            // query tiles per half
    static constexpr int NB = BC / 32;            // 32-key blocks per chunk
    static constexpr int NB0 = NB / 2;            // key blocks the first half reaches
    static constexpr int KS = DK / 32;            // 32-wide k-steps over d_k
    static constexpr int RT = DK / 16;            // 16-row tiles of d_k
    static constexpr int NVB = 32 * WS * 2 / FB;  // 1 KiB blocks of V per key block
    // P^T fragments the units carry: (u, kb) for u < NH, kb < NB0 with the
    // first half's V rows; u >= NH with each key block
    static constexpr int PU0 = NH;
    static constexpr int PU1 = SO ? 0 : NH;
    // unit layouts (bytes within a slot)
    static constexpr int QF_BYTES = NH * KS * FB;
    static constexpr int VP_PF = NB0 * NVB * FB;  // P^T after the V rows
    static constexpr int VP_BYTES = VP_PF + PU0 * NB0 * FB;
    static constexpr int KP_PF = RT * FB;         // P^T after the KF fragments
    static constexpr int KP_V = (RT + PU1) * FB;  // then the V rows
    static constexpr int KP_BYTES = KP_V + NVB * FB;
    static constexpr int SLOT = SO ? KP_BYTES : max3(QF_BYTES, VP_BYTES, KP_BYTES);
    static constexpr int NQ = SO ? 0 : 3;         // QF(h0), VP, QF(h1)
    static constexpr int NU = NQ + NB;            // units per chunk
    static constexpr int NSLOT = LDS_BYTES / SLOT < 4 ? LDS_BYTES / SLOT : 4;
    static constexpr int D = NSLOT - 1;           // units loaded ahead
    // Loads per wave of unit u of a chunk.  A unit is a list of segments of
    // 1 KiB blocks of one kind (QF; V, P^T; KF, P^T, V); wave w takes blocks
    // w, w + NWV, ... of each segment, and a segment's last round wraps
    // around (repeats load the same block into the same place), so every
    // wave issues the same loads and each load's kind is known at compile
    // time.
    __host__ __device__ static constexpr int rounds(int n) { return (n + NWV - 1) / NWV; }
    __host__ __device__ static constexpr int loads(int u) {
        return u >= NQ ? rounds(RT) + rounds(PU1) + rounds(NVB)
                       : u == 1 ? rounds(NB0 * NVB) + rounds(PU0 * NB0) : rounds(NH * KS);
    }
    // stores per wave after unit u: the outputs and GroupNorm partials of a half
    __host__ __device__ static constexpr int stores(int u) {
        return SO ? 0 : (u == 1 || u == NU - 1) ? 2 * NH : 0;
    }
    // memory operations a wave has issued after the loads of unit u when
    // unit u starts: the loads of the next D - 1 units and the stores after
    // units u - D .. u - 1 (before the first chunk of a run, dummy stores
    // stand in for those of the previous chunk's last unit)
    __host__ __device__ static constexpr int wait_count(int u) {
        int n = 0;
        for (int m = u + 1; m < u + D; ++m) n += loads(m % NU);
        for (int m = u - D; m < u; ++m) n += stores((m + NU) % NU);
        return n;
    }
    __host__ __device__ static constexpr int max_wait() {
        int n = 0;
        for (int u = 0; u < NU; ++u) n = wait_count(u) > n ? wait_count(u) : n;
        return n;
    }
    static_assert(SO || NU > D, "the stores of one chunk end lie within the wait window once");
    static_assert(NSLOT >= 3 && NSLOT * SLOT <= LDS_BYTES, "LDS ring");
    static_assert(NB0 >= 1 && 2 * NH == NKT, "query halves");
    static_assert(max_wait() <= 63, "vmcnt range");
};

template <int DK, int BC, bool SO>
__global__ __launch_bounds__(NWV * 64) void chunk_wide_kernel(MsrConst c, ChunkArgs a) {
    using C = WCfg<DK, BC, SO>;
    __shared__ __attribute__((aligned(1024))) char lds[C::NSLOT * C::SLOT];

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    // workgroup -> (pair, segment, slice): the slices of one (pair, segment)
    // get ids equal mod 8, i.e. run on the same XCD and share its L2
    const int npairs = c.B * c.H;
    int pair, seg, slice;
    {
        const int id = blockIdx.x, nps = npairs * a.nseg;
        int ps;
        if (nps % 8 == 0) {
            const int xcd = id & 7, j = id >> 3;
            ps = (j / a.NW2) * 8 + xcd;
            slice = j % a.NW2;
        } else {
            ps = id / a.NW2;
            slice = id % a.NW2;
        }
        pair = ps / a.nseg;
        seg = ps % a.nseg;
    }
    const int b = pair / c.H, h = pair % c.H;
    const int col0 = slice * WS;    // the slice's first value column
    const int wc0 = col0 + w * WC;  // this wave's first value column
    // this lane's state elements (rt, ct, r): row 16 rt + 4 g + r, column
    // wc0 + 16 ct + l16 of a [d_k][d_v] state
    const size_t sbase = (size_t)pair * DK * c.dv + wc0 + (size_t)(4 * g) * c.dv + l16;
    const size_t ebase = (size_t)pair * a.nseg * DK * c.dv + wc0 + (size_t)(4 * g) * c.dv + l16;
    const size_t estride = (size_t)DK * c.dv;
    auto sidx = [&](int rt, int ct, int r) __attribute__((always_inline)) { return (size_t)(16 * rt + r) * c.dv + 16 * ct; };
    if (SO && seg == 0) {
        // s_in set aside in the last segment's slot, for the full pass
        float *dst = a.segE + ebase + (size_t)(a.nseg - 1) * estride;
        for (int rt = 0; rt < C::RT; ++rt)
            for (int ct = 0; ct < CT; ++ct)
                for (int r = 0; r < 4; ++r) dst[sidx(rt, ct, r)] = a.s_in ? a.s_in[sbase + sidx(rt, ct, r)] : 0.f;
    }
    if (SO && seg == a.nseg - 1) return;  // the last segment's end state is not needed
    const int i0 = seg * a.seglen, i1 = i0 + a.seglen;
    const float lg = c.log2g[h];
    const int period = rescale_period(lg, BC);
    // the carried S^ is S gamma^(-BC ph); entering chunk i0 it has the phase
    // of chunk i0 - 1
    int ph = i0 == 0 ? 0 : (i0 - 1) % period;
    const int nch = c.T / BC;
    const size_t pc0 = (size_t)pair * nch;
    // buffer resources over this pair's fragments and this slice's V rows;
    // each lane adds its 16-byte offset
    const auto rq = rsrc(a.qf + pc0 * (C::NKT * C::KS * FE), (uint32_t)nch * C::NKT * C::KS * FB);
    const auto rk = rsrc(a.kf + pc0 * (C::RT * C::NB * FE), (uint32_t)nch * C::RT * C::NB * FB);
    const auto rp = rsrc(a.pf + pc0 * (C::NKT * C::NB * FE), (uint32_t)nch * C::NKT * C::NB * FB);
    const uint32_t loff = lane * 16;
    const uint32_t rowV = (uint32_t)c.H * c.dv * 2;  // bytes between tokens of V
    const auto rv = rsrc(a.v + ((size_t)b * c.T * c.H + h) * c.dv + col0, (uint32_t)(c.T - 1) * rowV + WS * 2);

    // V block vj (rows 2 vj, 2 vj + 1) of key block kb of chunk ci.  The
    // lane's offset is recomputed at each load (a few ALU operations) rather
    // than kept in registers for the whole loop.
    auto issue_v = [&](int ci, int kb, int vj, char *dst) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int r = 2 * vj + (ln >> 5);
        const uint32_t vo = (ln >> 5) * rowV + (((ln & 31) ^ vswz(r)) << 4);
        load_lds16(rv, vo, (uint32_t)(ci * BC + 32 * kb + 2 * vj) * rowV, dst);
    };
    // block r NWV + w of a segment of n blocks (wrapping in the last round)
    auto seg_block = [&](int r, int n) __attribute__((always_inline)) {
        return NWV * (r + 1) <= n ? NWV * r + w : (NWV * r + w) % n;
    };
    // the loads of unit U of chunk ci into the LDS slot dst
    auto issue = [&](int ci, auto UC, char *dst) __attribute__((always_inline)) {
        constexpr int U = decltype(UC)::value;
        ci = ci < nch ? ci : nch - 1;  // beyond the last chunk: in bounds, never read
        if constexpr (C::NQ > 0 && (U == 0 || U == 2)) {  // QF of query half U / 2
#pragma unroll
            for (int r = 0; r < C::rounds(C::NH * C::KS); ++r) {
                const int j = seg_block(r, C::NH * C::KS), u = (U / 2) * C::NH + j / C::KS, ks = j % C::KS;
                load_lds16(rq, loff, (uint32_t)((ci * C::NKT + u) * C::KS + ks) * FB, dst + j * FB);
            }
        } else if constexpr (C::NQ > 0 && U == 1) {  // V and P^T of the key blocks the first half reaches
#pragma unroll
            for (int r = 0; r < C::rounds(C::NB0 * C::NVB); ++r) {
                const int j = seg_block(r, C::NB0 * C::NVB);
                issue_v(ci, j / C::NVB, j % C::NVB, dst + j * FB);
            }
#pragma unroll
            for (int r = 0; r < C::rounds(C::PU0 * C::NB0); ++r) {
                const int f = seg_block(r, C::PU0 * C::NB0), u = f / C::NB0, kb = f % C::NB0;
                load_lds16(rp, loff, (uint32_t)((ci * C::NKT + u) * C::NB + kb) * FB, dst + C::VP_PF + f * FB);
            }
        } else {  // key block U - NQ: KF, the second half's P^T, V
            constexpr int kb = U - C::NQ;
#pragma unroll
            for (int r = 0; r < C::rounds(C::RT); ++r) {
                const int j = seg_block(r, C::RT);
                load_lds16(rk, loff, (uint32_t)((ci * C::RT + j) * C::NB + kb) * FB, dst + j * FB);
            }
#pragma unroll
            for (int r = 0; r < C::rounds(C::PU1); ++r) {
                const int f = seg_block(r, C::PU1), u = C::NKT - C::PU1 + f;
                load_lds16(rp, loff, (uint32_t)((ci * C::NKT + u) * C::NB + kb) * FB, dst + C::KP_PF + f * FB);
            }
#pragma unroll
            for (int r = 0; r < C::rounds(C::NVB); ++r) {
                const int vj = seg_block(r, C::NVB);
                issue_v(ci, kb, vj, dst + C::KP_V + vj * FB);
            }
        }
    };
    // unit N counted from unit 0 of chunk ci
    auto issue_n = [&](int ci, auto NC, char *dst) __attribute__((always_inline)) {
        constexpr int N = decltype(NC)::value;
        issue(ci + N / C::NU, std::integral_constant<int, N % C::NU>{}, dst);
    };

    f32x4 S[C::RT][CT];
    {
        const float gseg = exp2f((float)(BC * a.seglen) * lg);
        const float f0 = exp2f(-(float)(BC * ph) * lg);
        const float *sin = a.nseg > 1 ? a.segE + ebase + (size_t)(a.nseg - 1) * estride : a.s_in + sbase;
        const bool has_in = !SO && (a.nseg > 1 || a.s_in);
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[rt][ct][r] = has_in ? sin[sidx(rt, ct, r)] : 0.f;
        // earlier segments' end states (the prologue runs before the chunk
        // loop's fragments and output tiles are live, so a batch of loads may
        // take up to 128 registers)
        if (!SO) fold_segments<128>(S, a.segE + ebase, estride, seg, gseg, sidx);
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) S[rt][ct] = S[rt][ct] * f0;
    }
    __builtin_amdgcn_s_waitcnt(0);

    f32x4 Ot[CT][C::NH];  // O^T of the current query half
    const int64_t rp0 = (c.flags & MSR_FLAG_DECAY_ROWNORM) ? row_pos0(c, b) : 0;
    // this batch row's outputs from the wave's first column on, and its
    // GroupNorm partials from the wave's slice on
    const uint32_t obytes = (uint32_t)c.T * c.H * c.dv * 2;
    const auto ro = rsrc(a.o + (size_t)b * c.T * c.H * c.dv + wc0, obytes - wc0 * 2);
    // (the partials are written whether or not the caller asked for
    // GroupNorm, so that every chunk issues the same stores)
    const uint32_t sbytes = (uint32_t)c.T * c.H * a.NS * 8;
    const auto rs = rsrc(a.stats + (size_t)b * c.T * c.H * a.NS + wc0 / WC, sbytes - (wc0 / WC) * 8);

    // O^T = S^T Q~^T (.) xi for the query half in slot sl
    auto cross = [&](const char *sl) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            bf16x8 A[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    A[ct][r] = static_cast<__bf16>(S[2 * ks][ct][r]);
                    A[ct][4 + r] = static_cast<__bf16>(S[2 * ks + 1][ct][r]);
                }
#pragma unroll
            for (int u = 0; u < C::NH; ++u) {
                const bf16x8 B = *reinterpret_cast<const bf16x8 *>(sl + (u * C::KS + ks) * FB + loff);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    Ot[ct][u] = mfma16(A[ct], B, ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : Ot[ct][u]);
            }
            sched_fence();
        }
    };
    // V^T fragments of the 32 V rows at Vs
    auto read_v = [&](const char *Vs, bf16x8 (&bv)[CT]) __attribute__((always_inline)) {
        static_assert(CT == 2, "two column tiles per wave");
        const uint32_t base = lds_addr(Vs);
        uint32_t ad[CT][2];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int col = w * WC + 16 * ct + 4 * (l16 & 3);
            ad[ct][0] = base + voff(4 * g + (l16 >> 2), col);
            ad[ct][1] = base + voff(16 + 4 * g + (l16 >> 2), col);
        }
        s16x4 t[CT][2];
        lds_tr4(ad[0][0], ad[0][1], ad[1][0], ad[1][1], t[0][0], t[0][1], t[1][0], t[1][1]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bv[ct] = cat(t[ct][0], t[ct][1]);
    };
    // row factor, GroupNorm partials and the stores of query half hf of chunk
    // ci.  Lane (l16, g) holds row 16 u + l16, columns 16 ct + 4 g .. + 3 of
    // tile (ct, u).  Two lane swaps give each lane 8 consecutive columns of
    // its row -- after exchanging the upper half of the ct = 0 values with the
    // lower half of the ct = 1 values (permlane32_swap), then the odd 16-lane
    // rows of the first register with the even rows of the second
    // (permlane16_swap), lane (l16, g) holds columns 8 g .. 8 g + 7 -- so each
    // row leaves in one 64-byte piece per wave.  Offsets are formed here from
    // an opaque lane index rather than kept in registers across the loop.
    auto finish = [&](int hf, int ci) __attribute__((always_inline)) {
        static_assert(CT == 2, "two column tiles per wave");
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const uint32_t orow = (uint32_t)c.H * c.dv * 2;  // bytes between tokens of O
        const uint32_t olane = (ln & 15) * orow + (ln >> 4) * 16;
        const uint32_t srow = (uint32_t)c.H * a.NS * 8;  // bytes between tokens of the partials
        const uint32_t slane = (ln & 15) * srow;
#pragma unroll
        for (int u = 0; u < C::NH; ++u) {
            const int t0 = ci * BC + 16 * (hf * C::NH + u);  // first token of the tile
            if (c.flags & MSR_FLAG_DECAY_ROWNORM) {
                const float f = 1.f / decay_row_sum(rp0 + t0 + (ln & 15), lg);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Ot[ct][u] = Ot[ct][u] * f;
            }
            {
                float sum = 0.f;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) sum += Ot[ct][u][0] + Ot[ct][u][1] + Ot[ct][u][2] + Ot[ct][u][3];
                const float mean = sum_lane_groups(sum) * (1.f / WC);
                float m2 = 0.f;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m2 += (Ot[ct][u][r] - mean) * (Ot[ct][u][r] - mean);
                m2 = sum_lane_groups(m2);
                const u32x2 st2 = {__float_as_uint(mean), __float_as_uint(m2)};
                if ((ln >> 4) == 0)  // every lane group holds the row's statistics
                    __builtin_amdgcn_raw_buffer_store_b64(st2, rs, slane, (uint32_t)(t0 * c.H + h) * a.NS * 8, 0);
            }
            uint32_t x[2], y[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const auto p = __builtin_amdgcn_permlane32_swap(pack_bf16x2(Ot[0][u][2 * i], Ot[0][u][2 * i + 1]),
                                                                pack_bf16x2(Ot[1][u][2 * i], Ot[1][u][2 * i + 1]),
                                                                false, false);
                const auto q = __builtin_amdgcn_permlane16_swap(p[0], p[1], false, false);
                x[i] = q[0];
                y[i] = q[1];
            }
            const u32x4 v4 = {x[0], x[1], y[0], y[1]};
            __builtin_amdgcn_raw_buffer_store_b128(v4, ro, olane, (uint32_t)(t0 * c.H + h) * c.dv * 2, 0);
        }
    };
    // the first half's value product (unit 1)
    auto value0 = [&](const char *sl) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < C::NB0; ++kb) {
            bf16x8 bv[CT];
            read_v(sl + kb * C::NVB * FB, bv);
#pragma unroll
            for (int u = 2 * kb; u < C::NH; ++u) {
                const bf16x8 B = *reinterpret_cast<const bf16x8 *>(sl + C::VP_PF + (u * C::NB0 + kb) * FB + loff);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Ot[ct][u] = mfma16(bv[ct], B, Ot[ct][u]);
            }
        }
    };
    // key block kb: the state update and the second half's value product
    auto block = [&](auto KC, const char *sl, int ci) __attribute__((always_inline)) {
        constexpr int kb = decltype(KC)::value;
        if constexpr (kb == 0) {
            const int j = ci % period;
            if (j == 0) {
                const float f = exp2f((float)(BC * (1 + ph)) * lg);
#pragma unroll
                for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        S[rt][ct] = S[rt][ct] * f;
                        sched_fence();
                    }
            }
            ph = j;
        }
        bf16x8 bv[CT];
        read_v(sl + C::KP_V, bv);
        // KF fragments in groups of 2 rows, the next group read while the
        // current one multiplies (bounded register use)
        constexpr int GR = 2;
        bf16x8 kfr[2][GR];
#pragma unroll
        for (int i = 0; i < GR; ++i) kfr[0][i] = *reinterpret_cast<const bf16x8 *>(sl + i * FB + loff);
#pragma unroll
        for (int g0 = 0; g0 < C::RT; g0 += GR) {
            if (g0 + GR < C::RT) {
#pragma unroll
                for (int i = 0; i < GR; ++i)
                    kfr[((g0 / GR) + 1) & 1][i] = *reinterpret_cast<const bf16x8 *>(sl + (g0 + GR + i) * FB + loff);
            }
#pragma unroll
            for (int i = 0; i < GR; ++i)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    S[g0 + i][ct] = mfma16(kfr[(g0 / GR) & 1][i], bv[ct], S[g0 + i][ct]);
            sched_fence();
        }
        if constexpr (!SO) {
#pragma unroll
            for (int u = (2 * kb > C::NH ? 2 * kb : C::NH); u < C::NKT; ++u) {
                const bf16x8 B =
                    *reinterpret_cast<const bf16x8 *>(sl + C::KP_PF + (u - (C::NKT - C::PU1)) * FB + loff);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Ot[ct][u - C::NH] = mfma16(bv[ct], B, Ot[ct][u - C::NH]);
            }
        }
    };

    if (i1 > i0) {
        static_for<C::D>([&](auto NC) __attribute__((always_inline)) { issue_n(i0, NC, lds + decltype(NC)::value * C::SLOT); });
        // stand-ins for the stores of the previous chunk's last unit: stores
        // through an empty buffer range, which the hardware drops
        const auto rnull = rsrc(a.o, 0);
#pragma unroll
        for (int i = 0; i < C::stores(C::NU - 1); ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, rnull, loff, 0, 0);
    }
    int n = 0;  // units started so far: unit n sits in slot n % NSLOT
    for (int ci = i0; ci < i1; ++ci) {
        static_for<C::NU>([&](auto UC) __attribute__((always_inline)) {
            constexpr int U = decltype(UC)::value;
            wait_vm<C::wait_count(U)>();
            lds_barrier();
            issue(ci + (U + C::D) / C::NU, std::integral_constant<int, (U + C::D) % C::NU>{},
                  lds + ((n + C::D) % C::NSLOT) * C::SLOT);
            sched_fence();
            const char *sl = lds + (n % C::NSLOT) * C::SLOT;
            if constexpr (C::NQ > 0 && (U == 0 || U == 2)) {
                cross(sl);
            } else if constexpr (C::NQ > 0 && U == 1) {
                value0(sl);
                finish(0, ci);
            } else {
                block(std::integral_constant<int, U - C::NQ>{}, sl, ci);
                if constexpr (!SO && U == C::NU - 1) finish(1, ci);
            }
            sched_fence();
            ++n;
        });
    }
    // the loads of units past the end and the stores may still be in flight
    __builtin_amdgcn_s_waitcnt(0);

    if (SO || (a.s_out && seg == a.nseg - 1)) {
        const float f = exp2f((float)(BC * ph) * lg);
        float *dst = SO ? a.segE + ebase + (size_t)seg * estride : a.s_out + sbase;
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[sidx(rt, ct, r)] = S[rt][ct][r] * f;
    }
}

template <int DK, int BC>
hipError_t launch_wide(const MsrConst &c, const ChunkArgs &a, bool so, hipStream_t st) {
    const unsigned grid = (unsigned)(c.B * c.H * a.nseg * a.NW2);
    if (so) {
        hipLaunchKernelGGL((chunk_wide_kernel<DK, BC, true>), dim3(grid), dim3(NWV * 64), 0, st, c, a);
    } else {
        hipLaunchKernelGGL((chunk_wide_kernel<DK, BC, false>), dim3(grid), dim3(NWV * 64), 0, st, c, a);
    }
    return hipGetLastError();
}

}  // namespace

namespace msr {

bool chunk_wide_supported(int dk, int dv, int bc) {
    return (dk == 128 || dk == 256) && (bc == 64 || bc == 128) && dv % WS == 0;
}

hipError_t launch_chunk_wide(const MsrConst &c, const ChunkArgs &a, int bc, bool state_only, hipStream_t st) {
    if (!chunk_wide_supported(c.dk, c.dv, bc) || a.NW2 != c.dv / WS) return hipErrorInvalidValue;
    if (state_only && (a.nseg < 2 || !a.segE)) return hipErrorInvalidValue;
    switch (c.dk * 1000 + bc) {
    case 128064: return launch_wide<128, 64>(c, a, state_only, st);
    case 128128: return launch_wide<128, 128>(c, a, state_only, st);
    case 256064: return launch_wide<256, 64>(c, a, state_only, st);
    case 256128: return launch_wide<256, 128>(c, a, state_only, st);
    default: return hipErrorNotSupported;
    }
}

}  // namespace msr
