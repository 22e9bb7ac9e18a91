// msr_internal.hpp -- shared between the C-ABI layer (msr_api.cpp) and the
// HIP kernels: the per-call constant block and the launcher prototypes.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "msr.h"

// Per-call constants, passed BY VALUE as a kernel argument (about 2 KiB, far
// below the kernel-argument limit), so no host->device copy is ever needed.
struct MsrConst {
    int32_t B, T, H, dk, dv;
    int32_t chunk;     // chunk size b (T for the parallel form)
    int64_t pos0;      // absolute position of token 0
    const int64_t *pos_rows;  // device: per-batch-row start positions (NULL: pos0 for all)
    float scale;       // multiplies the rotated K
    float eps;         // GroupNorm epsilon
    uint32_t flags;    // MSR_FLAG_*
    int32_t ldqk;      // elements between (token, head) rows of the Q and K the
                       // MFMA prep kernel reads (0: d_k, i.e. packed rows)
    int32_t revqk;     // nonzero: that kernel takes Q and K in reverse time order
                       // (token t of a batch row reads token T-1-t)
    float gamma[MSR_MAX_HEADS];   // decay per head
    float log2g[MSR_MAX_HEADS];   // log2(gamma), computed in fp64 on the host
    float theta[MSR_MAX_DK / 2];  // rotation frequency per channel pair
};

// ---- launchers (defined in the .hip files); all enqueue on `st` ----------

// X [B][T][H][dk] (fp32 or bf16) -> Xr [B][H][T][dk] fp32, rotated at
// positions pos0 + t and multiplied by `factor`.
hipError_t launch_rotate(const MsrConst &c, int dtype, const void *X, float *Xr, float factor,
                         hipStream_t st);

// Generic state pass over chunks of size `chunk`:
//   chunk_states[pair][i] = state entering chunk i (optional),
//   s_out = state after the last chunk (optional).
hipError_t launch_generic_state(const MsrConst &c, int dtype, int chunk, const float *Kr,
                                const void *V, const float *s_in, float *s_out,
                                float *chunk_states, hipStream_t st);

// Generic output pass: intra-chunk product + cross-chunk term read from
// states + pair * pair_stride + chunk_index * chunk_stride (states may be
// NULL: no cross-chunk term), GroupNorm, store O.
hipError_t launch_generic_output(const MsrConst &c, int dtype, int chunk, const float *Qr,
                                 const float *Kr, const void *V, void *O, const float *states,
                                 int64_t pair_stride, int64_t chunk_stride, hipStream_t st);

// Recurrent form over c.T <= MSR_DECODE_MAX_T tokens per pair with one pass
// over the state: s_in (NULL: zeros) -> s_out (NULL: dropped; may equal
// s_in).  The single-token decode step, and short chunkwise/parallel calls.
constexpr int MSR_DECODE_MAX_T = 16;
hipError_t launch_decode(const MsrConst &c, int dtype, const void *q, const void *k,
                         const void *v, void *o, const float *s_in, float *s_out, hipStream_t st);

// s_out = s_in (or zeros when s_in is NULL); used for T == 0.
hipError_t launch_copy_state(const MsrConst &c, const float *s_in, float *s_out, hipStream_t st);

// ---- backward-pass element-wise kernels (k_backward.hip) -------------------
// (every x / y below is an MSR_F32 or MSR_BF16 array as its *_dtype says)
hipError_t launch_to_f32(int dtype, size_t n, const void *x, float *y, hipStream_t st);
// y = factor * R(sign * angle) x on token-major [B][T][H][dk] rows; with ylo
// (bf16 output only) y + ylo is a two-term bf16 split of the fp32 result;
// rev: row t of y comes from row T-1-t of x; x2 (bf16, x's layout) is added
// to x first (both: d_k a multiple of 8 only)
hipError_t launch_rotate_tok(const MsrConst &c, const void *x, int in_dtype, void *y, int out_dtype, float factor,
                             float sign, hipStream_t st, void *ylo = nullptr, int rev = 0,
                             const void *x2 = nullptr);
// GroupNorm backward per row of dv values: x = GroupNorm's input, dy = dL/d(output) -> dx
hipError_t launch_gn_backward(size_t rows, int dv, float eps, const void *x, int x_dtype, const void *dy,
                              int dy_dtype, void *dx, int out_dtype, hipStream_t st);
// y[b][t'][h][0:len] = x[b][t][h][col0:col0+len], t' = T-1-t when reverse
hipError_t launch_slice(int B, int T, int H, int d, int col0, int len, int reverse, const void *x, int in_dtype,
                        void *y, int out_dtype, hipStream_t st);
// y = x + (first ? 0 : y), y fp32
// Q/K/V projections (k_proj.hip): Y[i] = X W[i]^T for the three matrices, X
// [M][d_model], W[i] [n[i]][d_model], Y[i] [M][n[i]], all bf16; with rotate,
// Y[0] and Y[1] rotated at each token's position and Y[1] scaled by c.scale
hipError_t launch_proj(const MsrConst &c, int M, int d_model, const void *X, const void *const W[3],
                       void *const Y[3], const int n[3], int rotate, hipStream_t st);
// rows [B][T][H][d] times the row-normalised-decay factor of c at their positions
hipError_t launch_row_scale(const MsrConst &c, int d, const void *x, int in_dtype, void *y, int out_dtype,
                            hipStream_t st);
hipError_t launch_accumulate(size_t n, const void *x, int in_dtype, float *y, int first, hipStream_t st);
// states [B][H][d1][d2] scaled by gamma_h^power (in NULL -> zeros); transpose != 0 writes
// rows j0..j0+nj-1 of the transpose ([nj][d1] per pair)
hipError_t launch_state_op(const MsrConst &c, int d1, int d2, const float *in, float *out, int transpose,
                           float power, int j0, int nj, hipStream_t st);

// The fixed scratch array of msr_chunkwise_noalloc (k_static.hip): this
// device's copy, looked up once per device.
constexpr size_t MSR_STATIC_SCRATCH_BYTES = MSR_NOALLOC_SCRATCH_BYTES;
hipError_t static_scratch(void **ptr);

// The process-wide msr_exchange_mode (msr_set_exchange).
int exchange_mode();

// Measurement hook (msr_set_kernel_events): records the caller's events
// around the main kernel of a call on its stream.  No-ops when unset.
void main_kernel_begin(hipStream_t st);
void main_kernel_end(hipStream_t st);
// The caller's events (null when unset), and a launch of a call's main
// kernel that attaches them to the kernel's own dispatch (its start and end
// times) rather than recording them as separate commands around it.
hipEvent_t main_event_start();
hipEvent_t main_event_stop();
template <typename F, typename... Args>
inline void launch_main(F kern, dim3 grid, dim3 block, hipStream_t st, Args... args) {
    const hipEvent_t a = main_event_start(), b = main_event_stop();
    if (a && b)
        hipExtLaunchKernelGGL(kern, grid, block, 0u, st, a, b, 0u, args...);
    else
        hipLaunchKernelGGL(kern, grid, block, 0, st, args...);
}
