// k_chunk_mfma.hip -- bf16 MFMA path (not yet enabled).
#include "msr_mfma.hpp"

bool mfma_supported(const msr_problem *, int, int) { return false; }
size_t mfma_workspace_bytes(const msr_problem *, int, int) { return 0; }

hipError_t mfma_chunkwise(const MsrConst &, const msr_problem *, int, const void *, const void *,
                          const void *, void *, const float *, float *, void *, hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t mfma_parallel(const MsrConst &, const msr_problem *, const void *, const void *,
                         const void *, void *, const float *, float *, void *, hipStream_t) {
    return hipErrorNotSupported;
}
