// k_proj.hip -- the Q/K/V projections in front of multi-scale retention
// (jsqmd.com "From RoPE to Retention" s2: the input goes through linear
// layers to give Q, K and V, then Q and K are rotated):
//   Q~ = R(X Wq^T),  K~ = s R(X Wk^T),  V = X Wv^T
// X is [M = B T][d_model] bf16 and each W is [out features][d_model] bf16
// (the layout of a linear layer's weight), so both MFMA operands read
// d_model-contiguous rows.  One launch covers the three matrices: a bf16
// MFMA GEMM (16x16x32, fp32 accumulation) whose epilogue rotates the fp32
// results of Q and K by their tokens' positions and applies K's scale
// before the single rounding to bf16.  Outputs are [B][T][H][d], i.e. the
// [M][H d] GEMM result.
//
// Tiling: a workgroup of 8 waves computes a 256 x 256 output tile, wave
// (wm, wn) the 64 tokens wm and the 128 features wn of it as 4 x 8 MFMA
// tiles (128 accumulator registers).  Per 64-wide step of d_model the A (X)
// and B (W) tiles go from global memory straight into LDS (direct 16-byte
// loads, one step ahead into the other of two buffers); rows are 128 bytes
// with their 16-byte chunks XOR-swizzled by row, which the direct loads
// realise by choosing each lane's source chunk.  One wait and one barrier
// per step.  Rows past M or past a matrix's width are clamped on load and
// skipped on store.
#include "msr_device.hpp"

namespace {

using namespace msr;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64, NT = 512;
constexpr int ROWB = BK * 2;            // bytes per LDS tile row
constexpr int TILEB = BM * ROWB;        // bytes per LDS tile (32 KiB; BN == BM)
constexpr int LPW = TILEB / 1024 / 8;   // 1 KiB direct loads per wave per tile

struct ProjArgs {
    const uint16_t *x;
    const uint16_t *w[3];
    uint16_t *y[3];
    int n[3];      // output features of each matrix
    int nt[3];     // 256-column tiles of each matrix
    int M, K;      // tokens, d_model
    int mt;        // 256-row tiles
    int rotate;    // rotate (and scale) the Q and K results
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (the LDS address is wave-uniform)
__device__ __forceinline__ void load_lds16(const void *gptr, void *lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)gptr,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

__global__ __launch_bounds__(NT) void proj_gemm_kernel(MsrConst c, ProjArgs a) {
    __shared__ __attribute__((aligned(1024))) char As[2][TILEB];
    __shared__ __attribute__((aligned(1024))) char Bs[2][TILEB];

    // tile id -> (matrix, row tile, column tile).  Ids are dealt round-robin
    // over the 8 XCDs; each XCD takes a contiguous range of the tile order,
    // in which groups of 8 row tiles sweep the column tiles, so the tiles an
    // XCD runs together share A rows and B columns in its L2.
    const int total = a.mt * (a.nt[0] + a.nt[1] + a.nt[2]);
    const int per = (total + 7) / 8;
    const int id = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (id >= total) return;
    int mat = 0, rem = id;
    while (mat < 2 && rem >= a.mt * a.nt[mat]) rem -= a.mt * a.nt[mat++];
    const int ntm = a.nt[mat];
    const int grp = rem / (8 * ntm), in = rem % (8 * ntm);
    const int gm = min(8, a.mt - grp * 8);
    const int tm = grp * 8 + in % gm, tn = in / gm;
    const int m0 = tm * BM, n0 = tn * BN, N = a.n[mat];
    const uint16_t *W = a.w[mat];

    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int wm = wv >> 1, wn = wv & 1;

    // direct loads: wave wv fills 1 KiB blocks j = wv + 8 i of each tile, i.e.
    // rows 8 j .. 8 j + 7; lane l writes row 8 j + l / 8 at physical chunk
    // l % 8, so it reads the logical chunk (l % 8) ^ (row & 7)
    const char *ag[LPW];
    const char *bg[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int r = 8 * (wv + 8 * i) + (lane >> 3);
        const int ch = (lane & 7) ^ (r & 7);
        const int mr = min(m0 + r, a.M - 1), nr = min(n0 + r, N - 1);
        ag[i] = reinterpret_cast<const char *>(a.x + (size_t)mr * a.K) + ch * 16;
        bg[i] = reinterpret_cast<const char *>(W + (size_t)nr * a.K) + ch * 16;
    }
    auto issue = [&](int kt, int buf) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            load_lds16(ag[i] + (size_t)kt * ROWB, As[buf] + (wv + 8 * i) * 1024);
            load_lds16(bg[i] + (size_t)kt * ROWB, Bs[buf] + (wv + 8 * i) * 1024);
        }
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = a.K / BK;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) issue(kt + 1, buf ^ 1);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 fa[4], fb[8];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = *reinterpret_cast<const bf16x8 *>(As[buf] + swz(wm * 64 + 16 * i + l16, 4 * ks + g));
#pragma unroll
            for (int j = 0; j < 8; ++j)
                fb[j] = *reinterpret_cast<const bf16x8 *>(Bs[buf] + swz(wn * 128 + 16 * j + l16, 4 * ks + g));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(fb[j], fa[i], acc[i][j]);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the next tiles have landed in LDS
        __syncthreads();
    }

    // epilogue.  With the weights as the MFMA's first operand, the result
    // tile's rows are output features and its columns tokens: lane (l16, g)
    // of acc[i][j] holds token m0 + wm 64 + 16 i + l16 and features
    // n0 + wn 128 + 16 j + 4 g + r, r = 0..3 -- four consecutive features,
    // two rotation pairs, in one lane.
    const bool rot = a.rotate && mat < 2;
    const float fac = mat == 1 && a.rotate ? c.scale : 1.f;
    uint16_t *Y = a.y[mat];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 64 + 16 * i + l16;
        if (m >= a.M) continue;
        const int bb = m / c.T, t = m - bb * c.T;
        const int64_t pos = row_pos0(c, bb) + t;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = n0 + wn * 128 + 16 * j + 4 * g;
            if (n >= N) continue;
            float y[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            if (rot) {
                const int e = n % c.dk;  // feature within the head: pairs e/2, e/2 + 1
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    float cs, sn;
                    rot_cos_sin(pos, c.theta[e / 2 + q], cs, sn);
                    const float x0 = y[2 * q], x1 = y[2 * q + 1];
                    y[2 * q] = x0 * cs - x1 * sn;
                    y[2 * q + 1] = x1 * cs + x0 * sn;
                }
            }
            const bf16x2 p0 = {static_cast<__bf16>(y[0] * fac), static_cast<__bf16>(y[1] * fac)};
            const bf16x2 p1 = {static_cast<__bf16>(y[2] * fac), static_cast<__bf16>(y[3] * fac)};
            const uint2 v2 = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
            *reinterpret_cast<uint2 *>(Y + (size_t)m * N + n) = v2;
        }
    }
}

}  // namespace

hipError_t launch_proj(const MsrConst &c, int M, int d_model, const void *X, const void *const W[3],
                       void *const Y[3], const int n[3], int rotate, hipStream_t st) {
    ProjArgs a;
    a.x = static_cast<const uint16_t *>(X);
    a.M = M;
    a.K = d_model;
    a.mt = (M + BM - 1) / BM;
    a.rotate = rotate;
    int total = 0;
    for (int i = 0; i < 3; ++i) {
        a.w[i] = static_cast<const uint16_t *>(W[i]);
        a.y[i] = static_cast<uint16_t *>(Y[i]);
        a.n[i] = n[i];
        a.nt[i] = (n[i] + BN - 1) / BN;
        total += a.mt * a.nt[i];
    }
    if (total == 0) return hipSuccess;
    const unsigned grid = (unsigned)(((total + 7) / 8) * 8);
    hipLaunchKernelGGL(proj_gemm_kernel, dim3(grid), dim3(NT), 0, st, c, a);
    return hipGetLastError();
}
