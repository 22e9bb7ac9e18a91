/*
 * msr.h -- C ABI of libmsr.so: multi-scale retention (MSR) on one AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (pages cited by site and section):
 *   - Q is rotated by Theta and K by its conjugate with the rotate-every-two
 *     cos/sin shift (jsqmd.com "From RoPE to Retention", section 2, the
 *     theta_shift snippet).  Pair i = (x[2i], x[2i+1]) of a token at absolute
 *     position p becomes (x0 cos a - x1 sin a, x1 cos a + x0 sin a) with
 *     a = p * theta[i].  The same real rotation is applied to Q and K: their
 *     real dot product then depends only on the position difference, which
 *     is what the conjugate pairing provides.
 *   - Scores are scaled by d_k^-0.5 (same page, section 5).  The scale is
 *     folded into the rotated K, so the carried state holds scaled keys.
 *   - Decay mask D[n][m] = gamma_h^(n-m) for n >= m, else 0, one gamma per
 *     head (same page, section 3; aiqz.cc RetNet tutorial, "retention score
 *     and exponential decay", "multi-scale retention").
 *   - Three equivalent forms (jsqmd.com section 4; aiqz.cc "parallel",
 *     "recurrent" and "chunkwise" representations; b99b.cn QbitAI article):
 *       parallel   O = (Q~ K~^T (.) D) V  (+ gamma^(n+1) Q~ S_in)
 *       chunkwise  per chunk i of b tokens, local index j, token t:
 *                  O = (Q~_i K~_i^T (.) D_b) V_i + (Q~_i S_{i-1}) (.) xi,
 *                  xi_j = gamma^(j+1);
 *                  S_i = gamma^b S_{i-1} + K~_i^T (V_i (.) zeta),
 *                  zeta_t = gamma^(b-1-t)
 *       recurrent  S_n = gamma S_{n-1} + k~_n^T v_n ;  o_n = q~_n S_n
 *   - Each head's output row (d_v values of one token) goes through a
 *     GroupNorm with no affine: (x - mean) / sqrt(biased var + eps)
 *     (jsqmd.com section 5; b99b.cn, GroupNorm's scale invariance).
 *
 * Layouts (row-major, no padding):
 *   Q, K   [B][T][H][dk]      dtype of the problem (fp32 or bf16)
 *   V, O   [B][T][H][dv]      dtype of the problem
 *   state  [B][H][dk][dv]     always fp32
 *   For msr_recurrent_step T is 1: q, k are [B][H][dk], v, o are [B][H][dv].
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers; gamma and theta are HOST arrays
 *     read during the call.  The caller owns every buffer; the library keeps
 *     no pointer after it returns and allocates no device memory.
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without synchronising.  Buffers must stay
 *     valid until the stream has passed the call.
 *   - All validation happens before anything is launched; on a non-OK status
 *     nothing has been written.  msr_last_error() then describes the
 *     problem.  A failed launch returns MSR_ERR_HIP.  Device faults surface
 *     at the caller's next synchronisation.
 *   - Device pointers must be 16-byte aligned.  O must not overlap Q, K, V
 *     or the state; state_out may equal state_in.
 *   - Non-finite input values are not checked; they propagate.
 *   - Scratch memory only ever comes from the caller's workspace `ws`, sized
 *     by msr_workspace_size().  Calls that share a workspace must be ordered
 *     on one stream.
 *   - The library keeps no state apart from per-thread error text and the
 *     per-thread measurement hook, so calls from several host threads are
 *     safe when their buffers are distinct.
 */
#ifndef MSR_H
#define MSR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 6: msr_set_exchange; 5: MSR_FLAG_FUSED (4: msr_workspace_bytes, msr_chunkwise_noalloc; strong-decay routing; 3: MSR_FLAG_DECAY_ROWNORM,
 * msr_qkv_projection, msr_qkv_chunkwise; 2: pos_rows) */
#define MSR_ABI_VERSION 6
#define MSR_MAX_HEADS 128 /* H limit (per-head constants travel by value) */
#define MSR_MAX_DK 512    /* d_k limit (theta values travel by value) */
#define MSR_MAX_DV 1024   /* d_v limit */

typedef enum {
    MSR_OK = 0,
    MSR_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad parameter value */
    MSR_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes, b not dividing T */
    MSR_ERR_DTYPE = -3,       /* unknown dtype */
    MSR_ERR_UNSUPPORTED = -4, /* valid problem this build does not handle */
    MSR_ERR_WORKSPACE = -5,   /* workspace missing or too small */
    MSR_ERR_HIP = -6          /* a HIP runtime call or kernel launch failed */
} msr_status;

typedef enum { MSR_F32 = 0, MSR_BF16 = 1 } msr_dtype;

/*
 * flags.  NO_ROTATE and NO_GROUPNORM switch parts of the operation off (used
 * for staged checks).  DECAY_ROWNORM normalises each row of the decay matrix
 * to unit sum (jsqmd.com section 5, "normalisation strategy", which lists it
 * among the score normalisations without a formula): the row of the token
 * at absolute position p is divided by the sum of its decay weights over
 * every position the sequence has reached, sum_{j=0}^{p} gamma^j =
 * (1 - gamma^(p+1)) / (1 - gamma) (p + 1 when gamma = 1), so that a sequence
 * split over several calls, its state carried, gives the same outputs as one
 * call.  The factor multiplies the row's output before GroupNorm, which
 * therefore sees it only through eps.
 */
/*
 * SPLIT_SCORES (a precision option of the bf16 matrix-core path of
 * msr_chunkwise; other paths compute the scores in fp32 and ignore it): the
 * intra-chunk scores q~ . k~ are taken from two-term bf16 splits of the fp32
 * rotated Q and K (hi.hi + lo.hi + hi.lo) instead of their bf16 roundings.
 * A score much smaller than |q~||k~| otherwise loses its relative accuracy,
 * which GroupNorm amplifies on rows dominated by few tokens -- under strong
 * decay enough to reach the bf16 tolerance.  Calls in which any head has
 * gamma < 0.9 take this route without the flag, msr_parallel included (it
 * then runs as the equal chunkwise form with chunk 64, 128 or 256).  Costs a
 * rotation pass and three score products instead of one.
 */
/*
 * FUSED (a schedule option of the bf16 matrix-core path of msr_chunkwise,
 * same results to within the bf16 tolerance): the rotation, the intra-chunk
 * scores and, when d_v is 256, GroupNorm run inside the recurrence
 * workgroups, from Q and K staged in LDS, instead of in separate passes
 * through HBM.  It moves about half the bytes of the default schedule but
 * is slower on MI355X at the shapes measured (its per-chunk vector work and
 * workgroup barriers outweigh the traffic saved), so it is not the default.
 * Taken for bf16, d_k 128 or 256, chunk 64 or 128, d_v a multiple of 256,
 * without SPLIT_SCORES, DECAY_ROWNORM or a gamma below 0.9; ignored otherwise.
 */
enum {
    MSR_FLAG_NO_ROTATE = 1u,
    MSR_FLAG_NO_GROUPNORM = 2u,
    MSR_FLAG_DECAY_ROWNORM = 4u,
    MSR_FLAG_SPLIT_SCORES = 8u,
    MSR_FLAG_FUSED = 16u
};

/* forms, for msr_workspace_size */
enum {
    MSR_FORM_PARALLEL = 0,
    MSR_FORM_CHUNKWISE = 1,
    MSR_FORM_STEP = 2,
    MSR_FORM_BACKWARD = 3,
    MSR_FORM_QKV_CHUNKWISE = 4 /* msr_qkv_chunkwise */
};

typedef struct {
    int32_t B, T, H, dk, dv; /* dk even, 2..MSR_MAX_DK; dv 4..MSR_MAX_DV, multiple of 4 */
    int32_t dtype;           /* msr_dtype of Q, K, V, O */
    const float *gamma;      /* [host] H decays, each in (0, 1] */
    const float *theta;      /* [host] dk/2 frequencies, or NULL => 10000^(-2i/dk) */
    float scale;             /* 0 => dk^-0.5; multiplies the rotated K */
    float gn_eps;            /* GroupNorm epsilon, >= 0 (1e-5 is the usual value) */
    int64_t pos0;            /* absolute position of token 0 (>= 0) for the rotation */
    uint32_t flags;          /* MSR_FLAG_* */
    /* [device] B starting positions, one per batch row (8-byte aligned), or
     * NULL: row b's token t is at position pos_rows[b] + t instead of pos0 + t.
     * For batched serving, where each sequence is at its own position.  The
     * values must be >= 0 and stay below 2^40 - T; they are not checked (they
     * live on the device). */
    const int64_t *pos_rows;
} msr_problem;

/* Library version check: returns MSR_ABI_VERSION. */
int msr_abi_version(void);

/* Text describing the last non-OK status returned on this host thread. */
const char *msr_last_error(void);

/*
 * Workspace bytes needed by `form` (MSR_FORM_*) for problem p; `chunk` is
 * the chunk size b for MSR_FORM_CHUNKWISE and ignored otherwise.  Validates
 * p like the compute calls (pointer fields are not dereferenced except
 * gamma/theta) and writes *bytes only on MSR_OK.
 */
msr_status msr_workspace_size(const msr_problem *p, int32_t form, int32_t chunk,
                              size_t *bytes);

/*
 * The same figure as a return value: the workspace bytes `form` needs for p
 * (chunk as above).  Returns 0 both when no workspace is needed and when p
 * is invalid; in the second case msr_last_error() says why (so a caller that
 * must tell the two apart uses msr_workspace_size).
 */
size_t msr_workspace_bytes(const msr_problem *p, int32_t form, int32_t chunk);

/*
 * Parallel form over all T tokens of every (batch, head) pair
 * (jsqmd.com section 4.1; aiqz.cc "parallel representation"):
 *   O[n] = GN( sum_{m<=n} gamma^(n-m) (q~_n . k~_m) v_m + gamma^(n+1) q~_n S_in )
 *   state_out = gamma^T S_in + sum_m gamma^(T-1-m) k~_m^T v_m
 * state_in NULL means a zero incoming state; state_out NULL skips it.
 * Equal, up to rounding, to msr_chunkwise with chunk == T.
 */
msr_status msr_parallel(const msr_problem *p, const void *Q, const void *K, const void *V,
                        void *O, const float *state_in, float *state_out, void *ws,
                        size_t ws_bytes, void *hip_stream);

/*
 * Chunkwise-recurrent form with chunk size `chunk` >= 1 (jsqmd.com section
 * 4.3; aiqz.cc "chunkwise recurrence"): the intra-chunk parallel product plus
 * the decayed state carried across chunks, as in the header comment.  When
 * chunk does not divide T the last chunk holds the remaining T mod chunk
 * tokens (computed on the general-purpose path).  Same outputs and state as
 * msr_parallel up to rounding, for any chunk.
 */
msr_status msr_chunkwise(const msr_problem *p, int32_t chunk, const void *Q, const void *K,
                         const void *V, void *O, const float *state_in, float *state_out,
                         void *ws, size_t ws_bytes, void *hip_stream);

/*
 * msr_chunkwise without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and rules as
 * msr_chunkwise; the scratch memory comes from a fixed array of
 * MSR_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  The call itself allocates nothing.
 *   - A problem whose msr_workspace_size(p, MSR_FORM_CHUNKWISE, chunk) exceeds
 *     that size is rejected with MSR_ERR_WORKSPACE before anything runs.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (different streams, or different host threads) race and give
 *     wrong results.  Order them on one stream.
 */
#define MSR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
msr_status msr_chunkwise_noalloc(const msr_problem *p, int32_t chunk, const void *Q, const void *K,
                                 const void *V, void *O, const float *state_in, float *state_out,
                                 void *hip_stream);

/*
 * Backward pass of the chunkwise form (equivalently of the parallel form):
 * the gradients of a loss L through the rotation, the scale, the retention
 * products and GroupNorm (jsqmd.com sections 2, 4 and 5; aiqz.cc parallel and
 * chunkwise representations, differentiated).  Given dO = dL/dO [B][T][H][dv]
 * (dtype of Q) and dstate_out = dL/dstate_out [B][H][dk][dv] (fp32, NULL for
 * zero), writes dQ, dK [B][T][H][dk] and dV [B][T][H][dv] (dtype of Q) and,
 * when dstate_in is non-NULL, dL/dstate_in (fp32).  Q, K, V and state_in are
 * the forward call's inputs (state_in NULL: zero); the forward activations
 * are recomputed, nothing from the forward call is needed.  fp32 inputs
 * (and bf16 shapes the matrix-core kernels do not take) run in fp32
 * arithmetic; bf16 inputs with dv a multiple of 64 run the products as bf16
 * matrix-core tiles with fp32 accumulation, the query-key scores from
 * two-term bf16 splits of the rotated Q and K.  Needs dv <= MSR_MAX_DK (else
 * MSR_ERR_UNSUPPORTED) and a workspace of
 * msr_workspace_size(p, MSR_FORM_BACKWARD, chunk) bytes.  The outputs must not
 * overlap the inputs or each other.
 */
msr_status msr_chunkwise_backward(const msr_problem *p, int32_t chunk, const void *Q, const void *K,
                                  const void *V, const float *state_in, const void *dO,
                                  const float *dstate_out, void *dQ, void *dK, void *dV, float *dstate_in,
                                  void *ws, size_t ws_bytes, void *hip_stream);

/*
 * Q/K/V projections of the layer input, the step in front of retention
 * (jsqmd.com section 2: the input goes through linear layers to give Q, K
 * and V, then Q is rotated by Theta and K by its conjugate):
 *   Q = R(X Wq^T),  K = s R(X Wk^T),  V = X Wv^T
 * with the rotation R and the scale s (p->scale, 0 => dk^-0.5) of the forms,
 * applied to the fp32 products before the one rounding to bf16.  With
 * MSR_FLAG_NO_ROTATE in p->flags the plain products are written (no rotation,
 * no scale).  Q, K so produced feed the forms with MSR_FLAG_NO_ROTATE and
 * scale 1 (msr_qkv_chunkwise does exactly that).
 *   X  [B][T][d_model] bf16; Wq, Wk [H*dk][d_model], Wv [H*dv][d_model] bf16
 *      (a linear layer's weight layout: output features by input features);
 *   Q, K [B][T][H][dk], V [B][T][H][dv] bf16, written.
 * p->dtype must be MSR_BF16 (else MSR_ERR_UNSUPPORTED); d_model must be a
 * positive multiple of 64 and H*dk a multiple of 4 (else MSR_ERR_SHAPE).
 * p->gamma is not used.  Outputs must not overlap inputs or each other.
 * Needs no workspace.
 */
msr_status msr_qkv_projection(const msr_problem *p, int32_t d_model, const void *X, const void *Wq,
                              const void *Wk, const void *Wv, void *Q, void *K, void *V,
                              void *hip_stream);

/*
 * The projections above followed by the chunkwise form: O and the outgoing
 * state of msr_chunkwise(p, chunk, R(X Wq^T), X Wk^T, X Wv^T), the rotation
 * and scale applied once, in the projection.  Q~, K~ and V live in the
 * workspace: msr_workspace_size(p, MSR_FORM_QKV_CHUNKWISE, chunk) bytes.
 * Same argument rules as msr_qkv_projection and msr_chunkwise.
 */
msr_status msr_qkv_chunkwise(const msr_problem *p, int32_t chunk, int32_t d_model, const void *X,
                             const void *Wq, const void *Wk, const void *Wv, void *O,
                             const float *state_in, float *state_out, void *ws, size_t ws_bytes,
                             void *hip_stream);

/*
 * One recurrent decode step for every pair, p->T must be 1 and p->pos0 is
 * the absolute position of the token (or p->pos_rows[b] that of batch row
 * b's token, for sequences at different positions) (jsqmd.com section 4.2;
 * aiqz.cc "recurrent representation"):
 *   state <- gamma state + k~^T v   (in place, fp32)
 *   o      = GN(q~ state)           (uses the updated state)
 * Needs no workspace.
 */
msr_status msr_recurrent_step(const msr_problem *p, const void *q, const void *k,
                              const void *v, void *o, float *state, void *hip_stream);

/*
 * Measurement hook (optional).  When `start` and `stop` are non-NULL
 * hipEvent_t handles (created with timing), each later compute call made on
 * this host thread records them at the start and the end of its main kernel:
 * the chunk-recurrence kernel of msr_chunkwise, the output kernel of
 * msr_parallel, the kernel of msr_recurrent_step.  For the matrix-core
 * chunk and parallel kernels and the decode kernels the events are attached
 * to the kernel's own dispatch (hipExtLaunchKernel), so the hook adds no
 * commands to the stream; elsewhere they are recorded on the call's stream
 * right before and after the kernel.  The caller owns the events; NULL, NULL
 * switches the hook off.  The hook only records events: results are
 * unchanged.
 */
void msr_set_kernel_events(void *start, void *stop);

/*
 * How msr_chunkwise's matrix-core chunk kernel finishes GroupNorm when a row's
 * d_v columns are split over several workgroups (GroupNorm over the heads'
 * outputs: jsqmd.com section 3, aiqz.cc "gated multi-scale retention").
 * Process-wide; applies to every later call on any device.
 *   MSR_EXCHANGE_AUTO (the default): when the call's whole grid can be resident
 *     at once, the workgroups of a row exchange their partial statistics
 *     through device memory and each normalises its own columns, waiting for
 *     its peers (at most 10 s, then it proceeds with what it has).  Of calls
 *     that overlap on one device only one waits at a time (a device-wide
 *     claim that the waiting call hands back once all its workgroups have
 *     started); the others take the MSR_EXCHANGE_NO_WAIT route.
 *   MSR_EXCHANGE_OFF: never wait; a separate GroupNorm pass follows the chunk
 *     kernel (about 2 us slower on the 7B-sized layer).  For callers that keep
 *     kernels of their own spinning on the device alongside, which the
 *     exchange's waits could otherwise outlast.
 *   MSR_EXCHANGE_NO_WAIT: the route a call takes when another call holds the
 *     claim: it stores un-normalised rows, and the last of each (pair,
 *     segment)'s workgroups to finish normalises that segment's rows from the
 *     exchanged statistics (one workgroup per segment: slower).  Selectable
 *     so that the route can be checked on its own.
 * Returns MSR_ERR_INVALID_ARG (and changes nothing) for any other value.
 */
typedef enum { MSR_EXCHANGE_AUTO = 0, MSR_EXCHANGE_OFF = 1, MSR_EXCHANGE_NO_WAIT = 2 } msr_exchange_mode;
msr_status msr_set_exchange(int32_t mode);

#ifdef __cplusplus
}
#endif

#endif /* MSR_H */
