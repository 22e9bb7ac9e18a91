// msr_mfma.hpp -- entry points of the MFMA (bf16 matrix-core) path.
#pragma once

#include "msr_internal.hpp"

// True when the MFMA kernels handle this problem/form/chunk.
bool mfma_supported(const msr_problem *p, int form, int chunk);

// Workspace the MFMA path needs (0 when it is not used for this problem);
// split: the chunkwise form with split scores (low parts of Q~, K~ given)
size_t mfma_workspace_bytes(const msr_problem *p, int form, int chunk, bool split = false);

// Qlo, Klo (optional, both or neither): low parts of two-term bf16 splits of
// Q and K; the intra-chunk scores then take hi.hi + lo.hi + hi.lo
hipError_t mfma_chunkwise(const MsrConst &c, const msr_problem *p, int chunk, const void *Q,
                          const void *K, const void *V, void *O, const float *s_in, float *s_out,
                          void *ws, hipStream_t st, const void *Qlo = nullptr, const void *Klo = nullptr);

hipError_t mfma_parallel(const MsrConst &c, const msr_problem *p, const void *Q, const void *K,
                         const void *V, void *O, const float *s_in, float *s_out, void *ws,
                         hipStream_t st);
