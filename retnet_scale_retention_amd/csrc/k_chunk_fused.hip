// k_chunk_fused.hip -- the chunkwise forward in one kernel (bf16 MFMA):
// rotation, intra-chunk scores, decay mask, value product, inter-chunk term,
// state carry and GroupNorm statistics, straight from the caller's Q, K, V.
//
// Per chunk i of b tokens (jsqmd.com "From RoPE to Retention" s2, s3, s4.3
// and s5; aiqz.cc RetNet tutorial, "chunkwise recurrence"):
//   Q~ = R(p theta) Q,  K~ = R(p theta) K       (rotate-every-two, fp32)
//   O_i = GN( (Q~_i K~_i^T s (.) D) V_i + (Q~_i S_{i-1}) (.) xi ),  xi_j = gamma^(j+1)
//   S_i = gamma^b S_{i-1} + K~_i^T (V_i (.) zeta s),                 zeta_t = gamma^(b-1-t)
//
// Workgroup: 8 waves (two per SIMD) own one (batch-head pair, slice of 256
// value columns, segment of chunks).  Wave w owns columns 32 w .. 32 w + 31
// of the slice and keeps in MFMA accumulators
//   - its fp32 state S[d_k][32] (16x16 tiles: rows 16 rt + 4 g + r, column
//     16 ct + l16 of lane (l16, g)) for the whole segment;
//   - O^T[32][b/2] of one query half at a time (32 registers at b = 128);
//   - the chunk's V[b][32] as bf16 A-operand fragments (V^T, keys in the
//     order {4g..4g+3, 16+4g..16+4g+3} of lane group g in each 32-key block).
// LDS holds the chunk's rotated Q~ and K~ (b x d_k bf16 each, rows with
// XOR-swizzled 16-byte chunks), one 32-key block of V on its way into the
// registers, the masked scores P^T as B-operand fragments and a GroupNorm
// exchange area: 156 KiB at d_k = 256, b = 128.
//
// Per chunk:
//   P1  scores of the first query half (keys of its own blocks), O^T =
//       S^T Q~^T (.) xi for that half, + V^T P^T, GroupNorm statistics,
//       output rows stored; the half's Q~ rows are dead: the next chunk's
//       first-half Q rows are loaded into them;
//   P2  O^T = S^T Q~^T (.) xi for the second half (S still the old state),
//       then per 32-key block: that block's scores for the second half,
//       + V^T P^T, and the state update S += K~^T (V (.) zeta s) (the carried
//       state is S up to a power of gamma that changes every few chunks:
//       rescale_period).  The block's K~ rows and V
//       registers are then dead: the next chunk's K block is loaded into the
//       rows and its V block, staged in LDS, read into the registers.
//       GroupNorm statistics and stores of the second half; the next chunk's
//       second-half Q rows are loaded.
//   end  the next chunk's first-half Q rows and first K blocks are rotated
//       in place; its second-half rows and later K blocks are rotated at its
//       P2, so their loads have P1 to land.
// All loads are direct buffer -> LDS copies (16 bytes per lane).  Every wave
// issues the same memory operations in the same order each chunk, so each
// wait is one fixed vmcnt; a barrier then tells that every wave's copies
// have landed.  The transpose reads run as asm blocks with their own LDS
// wait (the compiler would otherwise wait for every copy in flight).
//
// GroupNorm: each wave forms every row's (mean, M2) over its 32 columns.
// With d_v = 256 (NORM) the eight waves' partials meet in LDS, every wave
// combines them (Chan's pairwise formula, equal counts) and the rows are
// normalised before the store; otherwise the partials are written for
// gn_finalize_kernel (d_v / 32 per row) and O holds the pre-norm values.
//
// Rotation: the rows of Q~ and K~ at one position share their angles, so one
// pass rotates both tiles' rows of a query half; a table in LDS holds each
// frequency's 2 theta / pi (fp64) and cos / sin theta.
//
// Segments: a state-only instantiation (SO) computes each segment's end
// state from a zero state (K and V only) for segments 0 .. nseg-2 and sets
// s_in aside in the last segment's slot; the full pass starts segment g from
// S_in(g) = gamma^(b seglen) S_in(g-1) + E_(g-1), S_in(0) = s_in.
#include <utility>

#include "msr_chunk.hpp"
#include "msr_device.hpp"

namespace {

using namespace msr;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lchar;  // LDS bytes (32-bit addresses)

constexpr int NWV = 8;        // waves per workgroup
constexpr int NTH = NWV * 64;
constexpr int WC = 32;        // value columns per wave
constexpr int WS = NWV * WC;  // value columns per workgroup
constexpr int CT = WC / 16;   // 16-column tiles per wave
constexpr int FB = 1024;      // bytes per operand fragment
constexpr int LDS_MAX = 163840;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const lchar *p) { return (uint32_t)(uintptr_t)p; }

template <class T>
__device__ __forceinline__ T lds_ld(const lchar *p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T *>(p);
}
template <class T>
__device__ __forceinline__ void lds_st(lchar *p, T v) {
    *reinterpret_cast<__attribute__((address_space(3))) T *>(p) = v;
}

__device__ __forceinline__ bf16x8 cat(s16x4 a, s16x4 b) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2 y = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, y);
}

// 2^x by the hardware exponential: no special handling of results below the
// fp32 normal range (they flush towards 0: a decay weight that small is 0
// to within the tolerance)
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// x[l] + x[l ^ 16] + x[l ^ 32] + x[l ^ 48] in every lane (gfx950 lane swaps)
__device__ __forceinline__ float sum_lane_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Eight LDS transpose reads (ds_read_b64_tr_b16: within each 16-lane group,
// lane j points at 4 consecutive bf16 of row r0 + j/4, columns c0 + 4 (j%4);
// lane i then receives column c0 + i of rows r0 .. r0 + 3), complete when
// this returns: the wait is in the same asm block, because the compiler
// would otherwise wait for every direct load in flight before each read.
__device__ __forceinline__ void lds_tr8(const uint32_t (&a)[8], s16x4 (&r)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}

__device__ __forceinline__ void lds_tr4(const uint32_t (&a)[4], s16x4 (&r)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
}

// Buffer resource over nbytes from base (raw access; out-of-range reads
// return zeros, out-of-range stores are dropped)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds + 16 l (lds wave-uniform)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, lchar *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, (int)voff, 0, 0,
                                             0);
}

// s_waitcnt vmcnt(N), the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS: this wave's LDS accesses are complete and no
// memory access moves across it; global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int N, class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// cos and sin of pos * theta (radians), given t4 = 2 theta / pi in fp64.  The
// angle in quarter turns, pos * t4, is reduced to the nearest whole number q
// plus a remainder in [-1/2, 1/2] (exact: the subtraction of q loses no
// bits), i.e. y in [-pi/4, pi/4] radians; sin and cos of y come from their
// Taylor series up to y^9 and y^10 (truncation below 2e-9 and 1.2e-10), and
// q mod 4 quarter turns then rotate the pair.
__device__ __forceinline__ void rot_cs(double pos, double t4, float &cs, float &sn) {
    const double qt = pos * t4;
    const double q = rint(qt);
    const float y = (float)(qt - q) * 1.57079633f;
    const float y2 = y * y;
    const float s = y * (1.f - y2 * (1.f / 6.f - y2 * (1.f / 120.f - y2 * (1.f / 5040.f - y2 * (1.f / 362880.f)))));
    const float c =
        1.f - y2 * (0.5f - y2 * (1.f / 24.f - y2 * (1.f / 720.f - y2 * (1.f / 40320.f - y2 * (1.f / 3628800.f)))));
    // quarter turns: (c, s) -> (-s, c) -> (-c, -s) -> (s, -c), without branches
    const int qq = (int)(q - 4.0 * floor(q * 0.25));
    const float a = (qq & 1) ? s : c, bb = (qq & 1) ? c : s;
    cs = (qq == 1 || qq == 2) ? -a : a;
    sn = (qq >= 2) ? -bb : bb;
}

// XOR swizzle of the 16-byte chunks of a Q~ / K~ row in LDS: a bijection of
// the 16 rows of a tile whose values for any 4 rows 4m .. 4m + 3 differ in bits
// 2-3, so that 16 rows read at one chunk (the row reads of the score and
// inter-chunk products) and 4 rows read at two adjacent chunks (the transpose
// reads of the state update) both touch distinct 16-byte bank groups
__host__ __device__ constexpr int qkswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// XOR swizzle of the 16-byte chunks of a V row in LDS (256 columns): the
// transpose reads of a 16-lane group (4 rows x 32 bytes) touch 8 different
// 16-byte bank groups
__host__ __device__ constexpr int vswz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int voff(int r, int col) {
    return r * (WS * 2) + ((((col >> 3) ^ vswz(r))) << 4) + (col & 7) * 2;
}

template <int DK, int BC>
struct FCfg {
    static constexpr int NKT = BC / 16;  // 16-token tiles per chunk
    static constexpr int NH = NKT / 2;   // query tiles per half
    static constexpr int NB = BC / 32;   // 32-key blocks per chunk
    static constexpr int NB0 = NB / 2;   // key blocks the first half reaches
    static constexpr int KS = DK / 32;   // 32-wide k-steps over d_k
    static constexpr int RT = DK / 16;   // 16-row tiles of the state
    static constexpr int CH = DK / 8;    // 16-byte chunks per Q~/K~ row
    static constexpr int ROWB = DK * 2;  // bytes per Q~/K~ row
    static constexpr int RPU = FB / ROWB;  // rows per 1 KiB copy unit
    // LDS layout
    static constexpr int Q_BYTES = BC * ROWB;
    static constexpr int K_BYTES = BC * ROWB;
    static constexpr int V_BYTES = 32 * WS * 2;  // one 32-key block of V
    static constexpr int P0_FRAGS = NB0 * NH;    // first half: (kb, u) slots
    static constexpr int P_BYTES = (P0_FRAGS > 2 * NH ? P0_FRAGS : 2 * NH) * FB;
    static constexpr int GN_BYTES = (BC / 2) * NWV * 8;
    static constexpr int TH_BYTES = (DK / 2) * 16;  // per frequency: 2 theta / pi (fp64), cos theta, sin theta
    // (the small areas first: their addresses fit the 16-bit offset field of
    // the LDS instructions, so no base address is kept in a register)
    static constexpr int OFF_P = 0;
    static constexpr int OFF_GN = OFF_P + P_BYTES;
    static constexpr int OFF_TH = OFF_GN + GN_BYTES;
    static constexpr int OFF_V = OFF_TH + TH_BYTES;
    static constexpr int OFF_Q = OFF_V + V_BYTES;
    static constexpr int OFF_K = OFF_Q + Q_BYTES;
    static constexpr int LDS = OFF_K + K_BYTES;
    // memory operations per wave: copies of a Q half, a K block, a V block
    static constexpr int NQ = (BC / 2) / RPU / NWV;
    static constexpr int NK = 32 / RPU / NWV;
    static constexpr int NV = V_BYTES / FB / NWV;
    static_assert(LDS <= LDS_MAX, "LDS budget");
    static_assert(NQ * RPU * NWV == BC / 2 && NK * RPU * NWV == 32 && NV * NWV * FB == V_BYTES, "copy units");
    static_assert(NB0 >= 1 && 2 * NH == NKT && NH <= 4 && CH >= 16 && 32 * NB0 == BC / 2, "shape");
};

// Vector memory operations a wave has issued after a given one, at the wait
// points of a chunk (full pass; the state-only pass has no Q copies and no
// stores).  Program order per chunk:
//   P1: stores(h0) ns, copies Q(next, h0) NQ
//   P2 (wait A) ... per block kb: K(next, kb) NK, (wait B kb), V(next, kb+1) NV
//   stores(h1) ns, copies Q(next, h1) NQ, (wait C)
// The stores of a query half are its NH output pieces, plus one store of the
// waves' GroupNorm partials when the rows are not normalised in the kernel.
template <int DK, int BC, bool SO, bool NORM>
struct FWait {
    using C = FCfg<DK, BC>;
    static constexpr int nq = SO ? 0 : C::NQ, ns = SO ? 0 : C::NH + (NORM ? 0 : 1);
    // A: Q(this, h1) (last op of the previous chunk) -> stores(h0) + Q(next, h0)
    static constexpr int A = ns + nq;
    // B kb: V(this-next, kb) is the op before K(next, kb) (kb >= 1); for kb = 0
    // it is the last block copy of the previous chunk
    static constexpr int B0 = ns + nq + ns + nq + C::NK;
    static constexpr int B1 = C::NK;
    // C: K(next, NB0 - 1) -> V(next, NB0), then K and V of blocks NB0.., stores(h1), Q(next, h1)
    static constexpr int Cw = C::NV + (C::NB - C::NB0) * (C::NK + C::NV) + ns + nq;
    static_assert(A < 64 && B0 < 64 && Cw < 64, "vmcnt range");
};

template <int DK, int BC, bool SO, bool NORM>
__global__ __launch_bounds__(NTH) void chunk_fused_kernel(MsrConst c, FusedArgs a) {
    using C = FCfg<DK, BC>;
    using WT = FWait<DK, BC, SO, NORM>;
    static_assert(!(SO && NORM), "the state-only pass writes no outputs");
    __shared__ __attribute__((aligned(1024))) char lds_arr[C::LDS];
    lchar *const lds = (lchar *)lds_arr;
    lchar *const Qt = lds + C::OFF_Q;
    lchar *const Kt = lds + C::OFF_K;
    lchar *const Vs = lds + C::OFF_V;
    lchar *const Ps = lds + C::OFF_P;
    lchar *const Gn = lds + C::OFF_GN;  // float2 [BC/2][NWV]
    lchar *const Th = lds + C::OFF_TH;  // rotation constants per frequency

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // The lane index is refreshed through an opaque asm at every phase, so
    // that the compiler recomputes lane-dependent values (addresses, decay
    // factors) where they are used instead of keeping every chunk-invariant
    // one in registers across the loop.
    int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4, tid = (int)threadIdx.x;
    auto refresh = [&]() __attribute__((always_inline)) {
        asm volatile("" : "+v"(lane));
        l16 = lane & 15;
        g = lane >> 4;
        tid = w * 64 + lane;
    };
    // workgroup -> (pair, segment, slice): the slices of one (pair, segment)
    // get ids equal mod 8, i.e. run on the same XCD and share the chunk's Q
    // and K in its L2
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
    const size_t pstate = (size_t)pair * DK * c.dv;
    const size_t estride = (size_t)DK * c.dv;
    const size_t ebase = (size_t)pair * a.nseg * estride;

    if (SO && seg == a.nseg - 1) {
        // the last segment's end state is not needed: its slot holds this
        // slice of s_in, which the full pass reads, so that s_out may
        // overwrite s_in in any workgroup order
        float *dst = a.segE + ebase + (size_t)seg * estride + col0;
        for (int i = tid; i < DK * WS; i += NTH) {
            const size_t o = (size_t)(i / WS) * c.dv + i % WS;
            dst[o] = a.s_in ? a.s_in[pstate + col0 + o] : 0.f;
        }
        return;
    }

    const int nch = c.T / BC;
    const int i0 = seg * a.seglen, i1 = i0 + a.seglen;  // this workgroup's chunks
    const float lg = c.log2g[h];
    const float sc = c.scale;
    // The workgroup's chunks are taken in runs of at most `period`.  Within a
    // run the carried state after the chunk with run index j is
    // S^ = S gamma^(-b (j+1)), so the update is a plain accumulation
    // S^ += gamma^(-b (j+1)) K~^T (V (.) zeta s), the factor riding on the V
    // operand, and the inter-chunk term of chunk j reads S_prev = S^ gamma^(b j)
    // through its row factor.  Between runs S^ is multiplied back to S, outside
    // the chunk loop (an update of the accumulators inside it makes the
    // register allocator spill them).  period is the largest run with
    // gamma^(-b period) <= 2^80: S^ and the V factors then stay far inside
    // the fp32 and bf16 ranges.
    int period;
    {
        const float per = (float)BC * -lg;  // -log2(gamma^b) >= 0
        const float m = per > 0.f ? 80.f / per : 1e9f;
        period = m >= (float)(1 << 30) ? (1 << 30) : (m < 1.f ? 1 : (int)m);
    }
    int ph = 0;  // run index of the current chunk
    const bool rot = !(c.flags & MSR_FLAG_NO_ROTATE);
    // position of the batch row's token 0 (uniform: kept in scalar registers)
    int64_t p0;
    {
        const int64_t v = row_pos0(c, b);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
        p0 = (int64_t)(((uint64_t)hi << 32) | lo);
    }
    const double p0d = (double)p0;

    // this batch row's Q, K, V, O, statistics as buffers
    const uint32_t qk_bytes = (uint32_t)c.T * c.H * DK * 2;
    const auto rq = rsrc(a.q + (size_t)b * c.T * c.H * DK, qk_bytes);
    const auto rk = rsrc(a.k + (size_t)b * c.T * c.H * DK, qk_bytes);
    const auto rv = rsrc(a.v + (size_t)b * c.T * c.H * c.dv, (uint32_t)c.T * c.H * c.dv * 2);
    const auto ro = rsrc(a.o + (size_t)b * c.T * c.H * c.dv, (uint32_t)c.T * c.H * c.dv * 2);
    const auto rnull = rsrc(a.o, 0);  // stores through it are dropped
    // the waves' GroupNorm partials (NP per row: slice * NWV + wave)
    const auto rst = (!NORM && a.stats && !(c.flags & MSR_FLAG_NO_GROUPNORM))
                         ? rsrc(a.stats + (size_t)b * c.T * c.H * a.NP, (uint32_t)c.T * c.H * a.NP * 8)
                         : rnull;

    // ---- copies (each wave issues an equal share of 1 KiB units) -----------
    // rows r0 .. r0 + NR - 1 of chunk ci's Q or K tile into tile rows r0..
    auto copy_rows = [&](auto NRC, __amdgpu_buffer_rsrc_t r, lchar *tile, int r0, int ci) __attribute__((always_inline)) {
        constexpr int NR = decltype(NRC)::value;
        constexpr int PER = NR / C::RPU / NWV;
        ci = ci < nch ? ci : nch - 1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int n = i * NWV + w;  // unit
            const int row = r0 + n * C::RPU + lane / C::CH;
            const int lchunk = (lane % C::CH) ^ qkswz(row & 15);
            const uint32_t t = (uint32_t)(ci * BC + row);
            dma16(r, ((t * c.H + h) * DK + lchunk * 8) * 2, tile + r0 * C::ROWB + n * FB);
        }
    };
    // 32-key block kb of chunk ci's V slice into the staging area
    auto copy_v = [&](int ci, int kb) __attribute__((always_inline)) {
        ci = ci < nch ? ci : nch - 1;
#pragma unroll
        for (int i = 0; i < C::NV; ++i) {
            const int n = i * NWV + w;
            const int row = n * 2 + (lane >> 5);
            const int lchunk = (lane & 31) ^ vswz(row);
            const uint32_t t = (uint32_t)(ci * BC + 32 * kb + row);
            dma16(rv, ((t * c.H + h) * c.dv + col0 + lchunk * 8) * 2, Vs + n * FB);
        }
    };

    // ---- rotation in place of rows r0 .. r0 + NR - 1 of chunk ci ----------
    // The rows of Q~ and K~ at one position share their angles: thread
    // (chunk c8, row group) rotates the 4 pairs of its 16-byte chunk of both
    // tiles (K~ only in the state-only pass) in a run of RPT rows; cos/sin of
    // the first row come from rot_cs, the later rows' by the angle-addition
    // formula with cos/sin of theta from the table in LDS.
    auto rotate = [&](auto NRC, int r0, int ci) __attribute__((always_inline)) {
        constexpr int NR = decltype(NRC)::value;
        constexpr int RPT = NR * C::CH / NTH;
        static_assert(RPT >= 1 && RPT * NTH == NR * C::CH, "rotation split");
        if (!rot) return;
        const int c8 = tid % C::CH, rg = tid / C::CH;
        const int rf = r0 + rg * RPT;
        const double pos = p0d + (double)(ci * BC + rf);
        float cs[4], sn[4], cd[4], sd[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x4 e = lds_ld<u32x4>(Th + (4 * c8 + p) * 16);
            const double t4 = __builtin_bit_cast(double, u32x2{e[0], e[1]});
            cd[p] = __uint_as_float(e[2]);
            sd[p] = __uint_as_float(e[3]);
            rot_cs(pos, t4, cs[p], sn[p]);
        }
        auto one = [&](lchar *px) __attribute__((always_inline)) {
            u32x4 x = lds_ld<u32x4>(px);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float x0 = lo_bf16(x[p]), x1 = hi_bf16(x[p]);
                x[p] = pack_bf16x2(x0 * cs[p] - x1 * sn[p], x1 * cs[p] + x0 * sn[p]);
            }
            lds_st(px, x);
        };
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int row = rf + r;
            const int off = row * C::ROWB + ((c8 ^ qkswz(row & 15)) << 4);
            if (!SO) one(Qt + off);
            one(Kt + off);
            if (r + 1 < RPT) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float cn = cs[p] * cd[p] - sn[p] * sd[p];
                    sn[p] = sn[p] * cd[p] + cs[p] * sd[p];
                    cs[p] = cn;
                }
            }
        }
    };

    // ---- the chunk's V in registers: Vw[kb][ct] = V^T A-operand fragment ----
    bf16x8 Vw[C::NB][CT];
    auto read_v = [&](bf16x8 (&dst)[CT]) __attribute__((always_inline)) {
        const uint32_t base = lds_addr(Vs);
        uint32_t ad[4];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int col = w * WC + 16 * ct + 4 * (l16 & 3);
            ad[2 * ct] = base + voff(4 * g + (l16 >> 2), col);
            ad[2 * ct + 1] = base + voff(16 + 4 * g + (l16 >> 2), col);
        }
        s16x4 t[4];
        lds_tr4(ad, t);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) dst[ct] = cat(t[2 * ct], t[2 * ct + 1]);
    };

    // ---- state -------------------------------------------------------------
    f32x4 S[C::RT][CT];
    {
        const float gseg = exp2f((float)(BC * a.seglen) * lg);  // gamma^(b seglen); runs start from the true state
        const float *sin_p = a.nseg > 1 ? a.segE + ebase + (size_t)(a.nseg - 1) * estride
                                        : (a.s_in ? a.s_in + pstate : nullptr);
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = 0.f;
                    if (!SO) {
                        const size_t o = (size_t)(16 * rt + 4 * g + r) * c.dv + wc0 + 16 * ct + l16;
                        x = sin_p ? sin_p[o] : 0.f;
                        for (int gg = 0; gg < seg; ++gg) x = x * gseg + a.segE[ebase + gg * estride + o];
                    }
                    S[rt][ct][r] = x;
                }
    }

    // rotation constants of each frequency (read after the prologue's barriers)
    if (rot && tid < DK / 2) {
        const double t4 = (double)c.theta[tid] * 0.63661977236758134;  // 2 / pi
        float cs1, sn1;
        rot_cs(1.0, t4, cs1, sn1);
        const u32x2 tb = __builtin_bit_cast(u32x2, t4);
        lds_st(Th + tid * 16, u32x4{tb[0], tb[1], __float_as_uint(cs1), __float_as_uint(sn1)});
    }

    // ---- prologue: chunk i0's Q, K and V, then the copies a previous chunk
    // would have left in flight (V block 0 of chunk i0 + 1, then stand-ins for
    // its second-half stores and the real second-half Q copy)
    if (!SO) copy_rows(std::integral_constant<int, BC / 2>{}, rq, Qt, 0, i0);
    copy_rows(std::integral_constant<int, BC>{}, rk, Kt, 0, i0);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    for (int kb = 0; kb < C::NB; ++kb) {
        copy_v(i0, kb);
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        static_for<C::NB>([&](auto KC) __attribute__((always_inline)) {
            if (decltype(KC)::value == kb) read_v(Vw[decltype(KC)::value]);
        });
        lds_barrier();
    }
    copy_v(i0 + 1, 0);
    if (!SO) {
#pragma unroll
        for (int i = 0; i < WT::ns; ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, rnull, lane * 4, 0, 0);
        copy_rows(std::integral_constant<int, BC / 2>{}, rq, Qt, BC / 2, i0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    rotate(std::integral_constant<int, BC / 2>{}, 0, i0);
    lds_barrier();

    // ---- output side: O^T of the current query half ------------------------
    f32x4 Ot[CT][C::NH];
    // P^T tile (key tile kt, query tile u) of the chunk, masked, decayed and
    // scaled, rounded to bf16 into half th of the B-operand fragment at frag
    auto score_tile = [&](int kt, int u, lchar *frag, int th) __attribute__((always_inline)) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const lchar *kr = Kt + (16 * kt + l16) * C::ROWB;
        const lchar *qr = Qt + (16 * u + l16) * C::ROWB;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int ch = (4 * ks + g) ^ qkswz(l16);
            const bf16x8 A = lds_ld<bf16x8>(kr + (ch << 4));
            const bf16x8 B = lds_ld<bf16x8>(qr + (ch << 4));
            acc = mfma16(A, B, acc);
            if (ks % 2 == 1) sched_fence();
        }
        const int j = 16 * u + l16;  // query (column of the tile)
        bf16x4 y;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = j - (16 * kt + 4 * g + r);
            y[r] = static_cast<__bf16>(d >= 0 ? acc[r] * sc * fexp2((float)d * lg) : 0.f);
        }
        lds_st(frag + 16 * lane + 8 * th, y);
    };
    // zeros into half th of a fragment (a key tile after every query of it)
    auto zero_tile = [&](lchar *frag, int th) __attribute__((always_inline)) {
        lds_st(frag + 16 * lane + 8 * th, u32x2{0u, 0u});
    };
    // O^T = S^T Q~^T (.) xi for query half hf
    auto inter = [&](int hf) __attribute__((always_inline)) {
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
            // channels {32 ks + 4 g .. + 3, 32 ks + 16 + 4 g .. + 3}: the rows
            // the two state tiles of the step leave in lane group g
            const int c1 = 4 * ks + (g >> 1), c2 = c1 + 2, in = (g & 1) * 8;
#pragma unroll
            for (int u = 0; u < C::NH; ++u) {
                const lchar *qr = Qt + (16 * (hf * C::NH + u) + l16) * C::ROWB;
                const u32x2 lo = lds_ld<u32x2>(qr + ((c1 ^ qkswz(l16)) << 4) + in);
                const u32x2 hi = lds_ld<u32x2>(qr + ((c2 ^ qkswz(l16)) << 4) + in);
                const bf16x8 B = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    Ot[ct][u] = mfma16(A[ct], B, ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : Ot[ct][u]);
            }
            sched_fence();
        }
#pragma unroll
        for (int u = 0; u < C::NH; ++u) {
            const float xi = fexp2((float)(16 * (hf * C::NH + u) + l16 + 1 + BC * ph) * lg);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) Ot[ct][u] = Ot[ct][u] * xi;
        }
    };
    // GroupNorm and the stores of query half hf of chunk ci
    auto finish = [&](int hf, int ci) __attribute__((always_inline)) {
        const int tq0 = ci * BC + 16 * hf * C::NH;  // first token of the half
        // (mean, M2) of each row over the wave's 32 columns; lane group g
        // keeps those of query tile u = g (row 16 g + l16)
        float pm = 0.f, pm2 = 0.f;
#pragma unroll
        for (int u = 0; u < C::NH; ++u) {
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
            pm = g == u ? mean : pm;
            pm2 = g == u ? m2 : pm2;
        }
        const int q = 16 * g + l16;
        if constexpr (NORM) {
            // The eight waves' partials of each row go to LDS (row q's 64
            // bytes, 16-byte slots permuted by q); after the barrier every
            // wave combines them (equal counts: Chan's pairwise formula) for
            // row lane mod (b/2) and takes row 16 u + l16's factors from lane
            // 16 u + l16.
            if (g < C::NH)
                lds_st(Gn + q * 64 + (((w >> 1) ^ (q & 3)) << 4) + (w & 1) * 8,
                       u32x2{__float_as_uint(pm), __float_as_uint(pm2)});
            lds_barrier();
            const int qr = lane & (BC / 2 - 1);
            float mw[NWV], m2w[NWV], mean = 0.f, m2 = 0.f;
#pragma unroll
            for (int i = 0; i < NWV / 2; ++i) {
                const f32x4 v = lds_ld<f32x4>(Gn + qr * 64 + ((i ^ (qr & 3)) << 4));
                mw[2 * i] = v[0];
                m2w[2 * i] = v[1];
                mw[2 * i + 1] = v[2];
                m2w[2 * i + 1] = v[3];
            }
#pragma unroll
            for (int i = 0; i < NWV; ++i) mean += mw[i];
            mean *= 1.f / NWV;
#pragma unroll
            for (int i = 0; i < NWV; ++i) m2 += m2w[i] + (float)WC * (mw[i] - mean) * (mw[i] - mean);
            const float rs = __builtin_amdgcn_rsqf(m2 * (1.f / WS) + c.eps);
            const float nb = -mean * rs;
#pragma unroll
            for (int u = 0; u < C::NH; ++u) {
                const int src = (16 * u + l16) * 4;
                const float ru = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(rs)));
                const float bu = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(nb)));
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Ot[ct][u][r] = Ot[ct][u][r] * ru + bu;
            }
        } else {
            // row q's partial (slice, wave) for the finishing pass; lane
            // groups past the half's tiles point past the buffer (dropped)
            const uint32_t t = (uint32_t)(tq0 + q);
            const uint32_t off = g < C::NH ? ((t * c.H + h) * a.NP + slice * NWV + w) * 8 : 0xfffffff0u;
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(pm), __float_as_uint(pm2)}, rst, off, 0, 0);
        }
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int u = 0; u < C::NH; ++u) {
            const uint32_t t = (uint32_t)(tq0 + 16 * u + l16);
            // two lane swaps give lane (l16, g) columns 8 g .. 8 g + 7 of its row
            uint32_t x[2], y[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const auto p = __builtin_amdgcn_permlane32_swap(pack_bf16x2(Ot[0][u][2 * i], Ot[0][u][2 * i + 1]),
                                                                pack_bf16x2(Ot[1][u][2 * i], Ot[1][u][2 * i + 1]),
                                                                false, false);
                const auto qq = __builtin_amdgcn_permlane16_swap(p[0], p[1], false, false);
                x[i] = qq[0];
                y[i] = qq[1];
            }
            const u32x4 v4 = {x[0], x[1], y[0], y[1]};
            const uint32_t off = (t * c.H + h) * c.dv * 2 + (uint32_t)wc0 * 2 + (uint32_t)(ln >> 4) * 16;
            __builtin_amdgcn_raw_buffer_store_b128(v4, ro, off, 0, 0);
            sched_fence();
        }
    };
    // the scores of the first query half: fragments (kb, u), kb < NB0, 2 kb <= u
    auto scores_h0 = [&]() __attribute__((always_inline)) {
        int n = 0;
#pragma unroll
        for (int kb = 0; kb < C::NB0; ++kb)
#pragma unroll
            for (int u = 2 * kb; u < C::NH; ++u)
#pragma unroll
                for (int th = 0; th < 2; ++th) {
                    const int kt = 2 * kb + th;
                    lchar *frag = Ps + (kb * C::NH + u) * FB;
                    if (kt <= u) {
                        if (n % NWV == w) score_tile(kt, u, frag, th);
                        ++n;
                    } else if ((kb * C::NH + u) % NWV == w) {
                        zero_tile(frag, th);
                    }
                }
    };
    // the scores of the second query half against key block kb (slot kb & 1)
    auto scores_h1 = [&](auto KC) __attribute__((always_inline)) {
        constexpr int kb = decltype(KC)::value;
        lchar *slot = Ps + (kb & 1) * C::NH * FB;
        int n = 0;
#pragma unroll
        for (int u = C::NH; u < C::NKT; ++u) {
            if (2 * kb > u) continue;
#pragma unroll
            for (int th = 0; th < 2; ++th) {
                const int kt = 2 * kb + th;
                lchar *frag = slot + (u - C::NH) * FB;
                if (kt <= u) {
                    if (n % NWV == w) score_tile(kt, u, frag, th);
                    ++n;
                } else if ((u - C::NH) % NWV == w) {
                    zero_tile(frag, th);
                }
            }
        }
    };
    // S += K~^T (V (.) zeta s) over key block kb
    auto state_block = [&](auto KC) __attribute__((always_inline)) {
        constexpr int kb = decltype(KC)::value;
        // B operand: the block's V (keys in the fragments' order) times
        // zeta_t s gamma^(-b (j+1)) = s gamma^(-1-t-b j)
        bf16x8 Bz[CT];
        {
            float z[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = 32 * kb + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
                z[e] = sc * fexp2((float)(BC - 1 - t - BC * (ph + 1)) * lg);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 8; ++e) Bz[ct][e] = static_cast<__bf16>((float)Vw[kb][ct][e] * z[e]);
        }
        // A operand: K~^T of the block by transpose reads, 2 row tiles at a time
        const uint32_t kbase = lds_addr(Kt);
        const int r1 = 32 * kb + 4 * g + (l16 >> 2);  // key rows of this lane's reads
        const int sw = qkswz(r1 & 15);                // (the same for r1 + 16)
#pragma unroll
        for (int q2 = 0; q2 < C::RT / 2; ++q2) {
            uint32_t ad[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rt = 2 * q2 + i;
                const int chk = ((2 * rt + ((l16 & 3) >> 1)) ^ sw) << 4;
                const int in = 8 * (l16 & 1);
                ad[2 * i] = kbase + r1 * C::ROWB + chk + in;
                ad[2 * i + 1] = kbase + (r1 + 16) * C::ROWB + chk + in;
            }
            s16x4 t[4];
            lds_tr4(ad, t);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bf16x8 A = cat(t[2 * i], t[2 * i + 1]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) S[2 * q2 + i][ct] = mfma16(A, Bz[ct], S[2 * q2 + i][ct]);
            }
            sched_fence();
        }
    };

    for (int r0 = i0; r0 < i1; r0 += period) {
      if (r0 > i0) {  // a run starts: S^ back to S
        const float f = exp2f((float)(BC * period) * lg);
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) S[rt][ct] = S[rt][ct] * f;
      }
      const int r1 = r0 + period < i1 ? r0 + period : i1;
      for (int ci = r0; ci < r1; ++ci) {
        ph = ci - r0;
        if (!SO) {
            // ------------------------------------------------ P1: first half
            refresh();
            scores_h0();
            lds_barrier();
            inter(0);
#pragma unroll
            for (int kb = 0; kb < C::NB0; ++kb) {
                static_for<C::NB>([&](auto KC) __attribute__((always_inline)) {
                    constexpr int k2 = decltype(KC)::value;
                    if (k2 != kb) return;
#pragma unroll
                    for (int u = 2 * k2; u < C::NH; ++u) {
                        const bf16x8 B = lds_ld<bf16x8>(Ps + (k2 * C::NH + u) * FB + 16 * lane);
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) Ot[ct][u] = mfma16(Vw[k2][ct], B, Ot[ct][u]);
                    }
                });
            }
            refresh();
            finish(0, ci);
            if (!NORM) lds_barrier();  // every wave is done with the half's Q~ rows
            refresh();
            copy_rows(std::integral_constant<int, BC / 2>{}, rq, Qt, 0, ci + 1);
        }
        // ---------------------------------------------------- P2: second half
        refresh();
        wait_vm<WT::A>();
        lds_barrier();
        rotate(std::integral_constant<int, BC / 2>{}, BC / 2, ci);
        lds_barrier();
        refresh();
        if (!SO) inter(1);
        static_for<C::NB>([&](auto KC) __attribute__((always_inline)) {
            constexpr int kb = decltype(KC)::value;
            refresh();
            if (!SO) {
                scores_h1(KC);
                lds_barrier();
                const lchar *slot = Ps + (kb & 1) * C::NH * FB;
#pragma unroll
                for (int u = C::NH; u < C::NKT; ++u) {
                    if (2 * kb > u) continue;
                    const bf16x8 B = lds_ld<bf16x8>(slot + (u - C::NH) * FB + 16 * lane);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Ot[ct][u - C::NH] = mfma16(Vw[kb][ct], B, Ot[ct][u - C::NH]);
                }
            }
            refresh();
            state_block(KC);
            lds_barrier();  // every wave is done with K~ block kb
            refresh();
            copy_rows(std::integral_constant<int, 32>{}, rk, Kt, 32 * kb, ci + 1);
            if (kb == 0)
                wait_vm<WT::B0>();
            else
                wait_vm<WT::B1>();
            lds_barrier();  // V block kb of the next chunk has landed
            read_v(Vw[kb]);
            lds_barrier();  // every wave has read it
            if (kb + 1 < C::NB)
                copy_v(ci + 1, kb + 1);
            else
                copy_v(ci + 2, 0);
        });
        if (!SO) {
            refresh();
            finish(1, ci);
            refresh();
            copy_rows(std::integral_constant<int, BC / 2>{}, rq, Qt, BC / 2, ci + 1);
        }
        // -------------------------------- end: the next chunk's first half
        wait_vm<WT::Cw>();
        lds_barrier();
        refresh();
        rotate(std::integral_constant<int, BC / 2>{}, 0, ci + 1);
        lds_barrier();
      }
    }

    // ---- the state --------------------------------------------------------
    float *dst = nullptr;
    if (SO)
        dst = a.segE + ebase + (size_t)seg * estride;
    else if (seg == a.nseg - 1 && a.s_out)
        dst = a.s_out + pstate;
    if (dst) {
        const float f = exp2f((float)(BC * (ph + 1)) * lg);  // S = S^ gamma^(b (j+1))
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(size_t)(16 * rt + 4 * g + r) * c.dv + wc0 + 16 * ct + l16] = S[rt][ct][r] * f;
    }
    // copies of chunks past the segment may still be in flight
    __builtin_amdgcn_s_waitcnt(0);
}

template <int DK, int BC>
hipError_t launch_dk_bc(const MsrConst &c, const FusedArgs &a, bool state_only, hipStream_t st) {
    const unsigned grid = (unsigned)(c.B * c.H * a.NW2 * a.nseg);
    // rows are normalised in the kernel when one slice spans d_v
    const bool norm = a.NS == 1 && !(c.flags & MSR_FLAG_NO_GROUPNORM);
    if (state_only)
        hipLaunchKernelGGL((chunk_fused_kernel<DK, BC, true, false>), dim3(grid), dim3(NTH), 0, st, c, a);
    else if (norm)
        hipLaunchKernelGGL((chunk_fused_kernel<DK, BC, false, true>), dim3(grid), dim3(NTH), 0, st, c, a);
    else
        hipLaunchKernelGGL((chunk_fused_kernel<DK, BC, false, false>), dim3(grid), dim3(NTH), 0, st, c, a);
    return hipGetLastError();
}

}  // namespace

namespace msr {

bool chunk_fused_supported(int dk, int dv, int bc) {
    return (dk == 128 || dk == 256) && (bc == 64 || bc == 128) && dv % WS == 0;
}

hipError_t launch_chunk_fused(const MsrConst &c, const FusedArgs &a, int bc, bool state_only, hipStream_t st) {
    if (state_only && (a.nseg < 2 || !a.segE)) return hipErrorInvalidValue;
    // (the kernel applies no row-normalised decay: such calls take the default schedule)
    if (c.flags & MSR_FLAG_DECAY_ROWNORM) return hipErrorInvalidValue;
    switch (c.dk * 1000 + bc) {
    case 128064: return launch_dk_bc<128, 64>(c, a, state_only, st);
    case 128128: return launch_dk_bc<128, 128>(c, a, state_only, st);
    case 256064: return launch_dk_bc<256, 64>(c, a, state_only, st);
    case 256128: return launch_dk_bc<256, 128>(c, a, state_only, st);
    default: return hipErrorNotSupported;
    }
}

}  // namespace msr
