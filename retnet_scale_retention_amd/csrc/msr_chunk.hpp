// msr_chunk.hpp -- what the chunkwise-form kernels share: the argument block
// of the chunk-recurrence kernels and the rescale period of the carried
// state, which prep_kernel's fragments and every chunk kernel must agree on.
#pragma once

#include "msr_device.hpp"

namespace msr {

// The chunk kernels carry S^ = S gamma^(-b j) instead of the state S, where
// j = (chunk index) mod m: within a run of m chunks the update is then a
// plain accumulation S^ += gamma^(-b j) K~^T (V (.) zeta) (the factor rides
// on the K~^T fragments), and S^ is multiplied by a power of gamma only when
// a run starts.  m is the largest period with gamma^(-b (m-1)) <= 2^40, so S^
// stays far from the fp32 range limits; gamma = 1 never rescales.
__device__ __forceinline__ int rescale_period(float lg, int bc) {
    const float per = (float)bc * -lg;  // -log2(gamma^b) >= 0
    const float m = per > 0.f ? 40.f / per + 1.f : 1e9f;
    return m >= (float)(1 << 30) ? (1 << 30) : (int)m;
}

struct ChunkArgs {
    const uint16_t *qf, *kf, *pf;  // fragments written by prep_kernel
    const uint16_t *v;
    uint16_t *o;
    const float *s_in;
    float *s_out;
    float2 *stats;  // [B*T*H][NS] (mean, M2) of each 64-column slice, when NS > 1 (or the exchange words)
    int NS;         // 64-column slices per pair (dv / 64)
    int NW2;        // workgroup slices per pair of the wide kernel (dv / 256), else NS
    int nseg, seglen;  // segments of seglen chunks per pair (nseg * seglen = T / b)
    float *segE;       // [pair][nseg][dk][dv] end state of each segment from a zero state
    int par;           // state-only pass of the parallel form: s_out = gamma^T s_in + sum of KF^T V
    // GroupNorm exchange between the value slices of a row (chunk_ws_kernel,
    // 2 <= NS <= 8): 16 + B H nseg counter words (eight ticket queues, the
    // call's mode, queues all started, and per (pair, segment) the finished
    // workgroups of a call that does not wait), null when the slices leave
    // (mean, M2) partials to gn_finalize_kernel instead.  The slices' words
    // live in `stats` (8 bytes each, [pair][chunk][tile][slice][16 rows]);
    // prep_kernel zeroes both.
    unsigned *xtick;
    unsigned xid;  // the call's nonzero id (ownership of the exchange)
};

// Argument block of the fused chunk kernel (k_chunk_fused.hip), which reads
// the caller's Q, K and V directly.
struct FusedArgs {
    const uint16_t *q, *k, *v;  // [B][T][H][d_k], [B][T][H][d_k], [B][T][H][d_v] bf16
    uint16_t *o;                // [B][T][H][d_v] bf16
    const float *s_in;
    float *s_out;
    float2 *stats;  // [B*T*H][NP] (mean, M2) of each wave's 32 columns (NS > 1)
    int NS;         // 256-column slices per pair (d_v / 256)
    int NW2;        // workgroup slices per pair (= NS)
    int NP;         // GroupNorm partials per row (d_v / 32)
    int nseg, seglen;  // segments of seglen chunks per pair
    float *segE;       // [pair][nseg][dk][dv] segment end states from a zero state
};

// The fused chunk kernel takes d_k 128 or 256, b 64 or 128, d_v a multiple
// of 256.
bool chunk_fused_supported(int dk, int dv, int bc);

// Launches it over pairs x a.NW2 x a.nseg workgroups: the state-only pass
// (segment end states) or the full pass.
hipError_t launch_chunk_fused(const MsrConst &c, const FusedArgs &a, int bc, bool state_only, hipStream_t st);

// Problem flag set only on the library's own sub-problems (the public entry
// points reject it like any unknown flag): keep the chunk recurrence on the
// 64-column kernels.  The backward pass sets it on its retention calls, for
// which those kernels are faster (they need no segment end states).
constexpr uint32_t kFlagNoWide = 1u << 31;

// The wide-slice chunk kernel (k_chunk_wide.hip): true when it can take
// this shape (d_k 128 or 256, b 64 or 128, d_v a multiple of 256).
bool chunk_wide_supported(int dk, int dv, int bc);

// Launches the wide-slice chunk kernel over pairs x a.NW2 x a.nseg
// workgroups: the state-only pass (segment end states) or the full pass.
hipError_t launch_chunk_wide(const MsrConst &c, const ChunkArgs &a, int bc, bool state_only, hipStream_t st);

}  // namespace msr
