"""MI355X-native multi-scale retention (RetNet MSR): parallel, chunkwise and
recurrent-step forms as hand-written HIP kernels behind the C ABI of
libmsr.so (include/msr.h).  This package is the thin Python binding."""
from .msr import (MSR_BF16, MSR_F32, MSR_FLAG_DECAY_ROWNORM, MSR_FLAG_NO_GROUPNORM, MSR_FLAG_NO_ROTATE,  # noqa: F401
                  MSR_FLAG_FUSED, MSR_FLAG_SPLIT_SCORES, MSR_EXCHANGE_AUTO, MSR_EXCHANGE_NO_WAIT, MSR_EXCHANGE_OFF,
                  MSR_FORM_BACKWARD, MSR_FORM_CHUNKWISE, MSR_FORM_PARALLEL, MSR_FORM_QKV_CHUNKWISE,
                  MSR_FORM_STEP, NOALLOC_SCRATCH_BYTES, MsrError, load, msr_chunkwise, msr_chunkwise_backward,
                  msr_chunkwise_noalloc, msr_parallel,
                  msr_qkv_chunkwise, msr_qkv_projection, msr_recurrent_step,
                  set_exchange, set_kernel_events,
                  workspace_size)
