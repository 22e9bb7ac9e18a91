// msr_api.cpp -- the C ABI of libmsr.so (declared in include/msr.h):
// argument validation, per-call constants, workspace carving and dispatch
// to the HIP kernels.  Validation completes before the first launch, so a
// non-OK status never leaves partial results behind.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "msr_internal.hpp"
#include "msr_mfma.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

msr_status fail(msr_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(int dtype) { return dtype == MSR_BF16 ? 2 : 4; }

// Checks the problem description.  `T1` requires T == 1 (decode step).
msr_status check_problem(const msr_problem *p, bool T1) {
    if (!p) return fail(MSR_ERR_INVALID_ARG, "problem pointer is NULL");
    if (p->dtype != MSR_F32 && p->dtype != MSR_BF16)
        return fail(MSR_ERR_DTYPE, "dtype %d is neither MSR_F32 (0) nor MSR_BF16 (1)", p->dtype);
    if (p->B < 0 || p->T < 0) return fail(MSR_ERR_SHAPE, "B=%d and T=%d must be >= 0", p->B, p->T);
    if (T1 && p->T != 1) return fail(MSR_ERR_SHAPE, "a decode step needs T == 1 (got %d)", p->T);
    if (p->H < 1 || p->H > MSR_MAX_HEADS)
        return fail(MSR_ERR_SHAPE, "H=%d outside 1..%d", p->H, MSR_MAX_HEADS);
    if (p->dk < 2 || p->dk > MSR_MAX_DK || (p->dk & 1))
        return fail(MSR_ERR_SHAPE, "dk=%d must be even and in 2..%d", p->dk, MSR_MAX_DK);
    if (p->dv < 4 || p->dv > MSR_MAX_DV || (p->dv & 3))
        return fail(MSR_ERR_SHAPE, "dv=%d must be a multiple of 4 in 4..%d", p->dv, MSR_MAX_DV);
    if ((int64_t)p->B * p->H > 65535)
        return fail(MSR_ERR_SHAPE, "B*H=%lld exceeds 65535", (long long)p->B * p->H);
    if (!p->gamma) return fail(MSR_ERR_INVALID_ARG, "gamma is NULL");
    for (int h = 0; h < p->H; ++h) {
        const float g = p->gamma[h];
        if (!(g > 0.f && g <= 1.f)) return fail(MSR_ERR_INVALID_ARG, "gamma[%d]=%g not in (0, 1]", h, g);
    }
    if (p->theta)
        for (int i = 0; i < p->dk / 2; ++i)
            if (!std::isfinite(p->theta[i]))
                return fail(MSR_ERR_INVALID_ARG, "theta[%d] is not finite", i);
    if (!std::isfinite(p->scale)) return fail(MSR_ERR_INVALID_ARG, "scale is not finite");
    if (!(p->gn_eps >= 0.f) || !std::isfinite(p->gn_eps))
        return fail(MSR_ERR_INVALID_ARG, "gn_eps=%g must be finite and >= 0", p->gn_eps);
    if (p->pos0 < 0) return fail(MSR_ERR_INVALID_ARG, "pos0=%lld must be >= 0", (long long)p->pos0);
    if (p->pos0 > ((int64_t)1 << 40) - p->T)
        return fail(MSR_ERR_INVALID_ARG, "positions beyond 2^40 are not supported");
    if (p->pos_rows && (reinterpret_cast<uintptr_t>(p->pos_rows) & 7u))
        return fail(MSR_ERR_INVALID_ARG, "pos_rows is not 8-byte aligned");
    if (p->flags & ~(uint32_t)(MSR_FLAG_NO_ROTATE | MSR_FLAG_NO_GROUPNORM))
        return fail(MSR_ERR_INVALID_ARG, "unknown flag bits 0x%x", p->flags);
    return MSR_OK;
}

MsrConst make_const(const msr_problem *p, int chunk) {
    MsrConst c{};
    std::memset(&c, 0, sizeof(c));
    c.B = p->B;
    c.T = p->T;
    c.H = p->H;
    c.dk = p->dk;
    c.dv = p->dv;
    c.chunk = chunk;
    c.pos0 = p->pos0;
    c.pos_rows = p->pos_rows;
    c.scale = p->scale != 0.f ? p->scale : (float)(1.0 / std::sqrt((double)p->dk));
    c.eps = p->gn_eps;
    c.flags = p->flags;
    for (int h = 0; h < p->H; ++h) {
        c.gamma[h] = p->gamma[h];
        c.log2g[h] = (float)std::log2((double)p->gamma[h]);
    }
    for (int i = 0; i < p->dk / 2; ++i)
        c.theta[i] = p->theta ? p->theta[i]
                              : (float)std::pow(10000.0, -2.0 * (double)i / (double)p->dk);
    return c;
}

// ---- workspace plans --------------------------------------------------------
// generic path: [Q~ fp32][K~ fp32][chunk states fp32 (chunkwise only)]
struct GenericPlan {
    size_t qr = 0, kr = 0, states = 0, total = 0;
};

GenericPlan generic_plan(const msr_problem *p, int form, int chunk) {
    GenericPlan g;
    const size_t tok = (size_t)p->B * p->T * p->H * p->dk * sizeof(float);
    g.qr = 0;
    g.kr = round_up(tok);
    g.states = g.kr + round_up(tok);
    g.total = g.states;
    if (form == MSR_FORM_CHUNKWISE && chunk > 0)  // a partial last chunk counts as a chunk
        g.total += round_up((size_t)p->B * p->H * ((p->T + chunk - 1) / chunk) * p->dk * p->dv * sizeof(float));
    return g;
}

msr_status check_tensors(const msr_problem *p, const void *Q, const void *K, const void *V,
                         const void *O, const float *s_in, const float *s_out) {
    const bool any = (size_t)p->B * p->T > 0;
    if (any && (!Q || !K || !V || !O)) return fail(MSR_ERR_INVALID_ARG, "Q, K, V and O must be non-NULL");
    const void *ptrs[6] = {Q, K, V, O, s_in, s_out};
    const char *names[6] = {"Q", "K", "V", "O", "state_in", "state_out"};
    for (int i = 0; i < 6; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(MSR_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    if (O && (O == Q || O == K || O == V))
        return fail(MSR_ERR_INVALID_ARG, "O must not alias Q, K or V");
    return MSR_OK;
}

msr_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MSR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MSR_OK;
}

}  // namespace

void main_kernel_begin(hipStream_t st) {
    if (g_ev_start) (void)hipEventRecord(g_ev_start, st);
}

void main_kernel_end(hipStream_t st) {
    if (g_ev_stop) (void)hipEventRecord(g_ev_stop, st);
}

extern "C" {

int msr_abi_version(void) { return MSR_ABI_VERSION; }

void msr_set_kernel_events(void *start, void *stop) {
    g_ev_start = static_cast<hipEvent_t>(start);
    g_ev_stop = static_cast<hipEvent_t>(stop);
}

const char *msr_last_error(void) { return g_err; }

msr_status msr_workspace_size(const msr_problem *p, int32_t form, int32_t chunk, size_t *bytes) {
    if (!bytes) return fail(MSR_ERR_INVALID_ARG, "bytes pointer is NULL");
    msr_status s = check_problem(p, form == MSR_FORM_STEP);
    if (s != MSR_OK) return s;
    if (form == MSR_FORM_STEP) {
        *bytes = 0;
        return MSR_OK;
    }
    if (form == MSR_FORM_CHUNKWISE) {
        if (chunk < 1) return fail(MSR_ERR_SHAPE, "chunk=%d must be >= 1", chunk);
    } else if (form != MSR_FORM_PARALLEL) {
        return fail(MSR_ERR_INVALID_ARG, "unknown form %d", form);
    }
    size_t need = generic_plan(p, form, chunk).total;
    const size_t mf = mfma_workspace_bytes(p, form, chunk);
    if (mf > need) need = mf;
    *bytes = need;
    return MSR_OK;
}

msr_status msr_parallel(const msr_problem *p, const void *Q, const void *K, const void *V,
                        void *O, const float *state_in, float *state_out, void *ws,
                        size_t ws_bytes, void *hip_stream) {
    msr_status s = check_problem(p, false);
    if (s != MSR_OK) return s;
    if ((s = check_tensors(p, Q, K, V, O, state_in, state_out)) != MSR_OK) return s;
    size_t need = 0;
    if ((s = msr_workspace_size(p, MSR_FORM_PARALLEL, 0, &need)) != MSR_OK) return s;
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(MSR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
    if (ws && !aligned16(ws)) return fail(MSR_ERR_INVALID_ARG, "ws is not 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const MsrConst c = make_const(p, p->T);
    if (p->B == 0) return MSR_OK;
    if (p->T == 0) return hip_status(launch_copy_state(c, state_in, state_out, st), "copy state");

    if (mfma_supported(p, MSR_FORM_PARALLEL, p->T))
        return hip_status(mfma_parallel(c, p, Q, K, V, O, state_in, state_out, ws, st), "mfma parallel");
    if (p->T <= MSR_DECODE_MAX_T) {  // a few tokens: the recurrence, one pass over the state
        main_kernel_begin(st);
        const hipError_t e = launch_decode(c, p->dtype, Q, K, V, O, state_in, state_out, st);
        main_kernel_end(st);
        return hip_status(e, "short parallel");
    }

    const GenericPlan g = generic_plan(p, MSR_FORM_PARALLEL, p->T);
    char *w = static_cast<char *>(ws);
    float *qr = reinterpret_cast<float *>(w + g.qr), *kr = reinterpret_cast<float *>(w + g.kr);
    hipError_t e = launch_rotate(c, p->dtype, Q, qr, 1.f, st);
    if (e == hipSuccess) e = launch_rotate(c, p->dtype, K, kr, c.scale, st);
    // outputs first: they read state_in, which state_out may overwrite
    if (e == hipSuccess) {
        main_kernel_begin(st);
        e = launch_generic_output(c, p->dtype, p->T, qr, kr, V, O, state_in,
                                  (int64_t)p->dk * p->dv, 0, st);
        main_kernel_end(st);
    }
    if (e == hipSuccess && state_out)
        e = launch_generic_state(c, p->dtype, p->T, kr, V, state_in, state_out, nullptr, st);
    return hip_status(e, "generic parallel");
}

msr_status msr_chunkwise(const msr_problem *p, int32_t chunk, const void *Q, const void *K,
                         const void *V, void *O, const float *state_in, float *state_out,
                         void *ws, size_t ws_bytes, void *hip_stream) {
    msr_status s = check_problem(p, false);
    if (s != MSR_OK) return s;
    if ((s = check_tensors(p, Q, K, V, O, state_in, state_out)) != MSR_OK) return s;
    size_t need = 0;
    if ((s = msr_workspace_size(p, MSR_FORM_CHUNKWISE, chunk, &need)) != MSR_OK) return s;
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(MSR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
    if (ws && !aligned16(ws)) return fail(MSR_ERR_INVALID_ARG, "ws is not 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const MsrConst c = make_const(p, chunk);
    if (p->B == 0) return MSR_OK;
    if (p->T == 0) return hip_status(launch_copy_state(c, state_in, state_out, st), "copy state");

    if (mfma_supported(p, MSR_FORM_CHUNKWISE, chunk))
        return hip_status(mfma_chunkwise(c, p, chunk, Q, K, V, O, state_in, state_out, ws, st),
                          "mfma chunkwise");
    if (p->T <= MSR_DECODE_MAX_T) {  // a few tokens: one pass over the state (the result is independent of b)
        main_kernel_begin(st);
        const hipError_t e = launch_decode(c, p->dtype, Q, K, V, O, state_in, state_out, st);
        main_kernel_end(st);
        return hip_status(e, "short chunkwise");
    }

    const GenericPlan g = generic_plan(p, MSR_FORM_CHUNKWISE, chunk);
    char *w = static_cast<char *>(ws);
    float *qr = reinterpret_cast<float *>(w + g.qr), *kr = reinterpret_cast<float *>(w + g.kr);
    float *cs = reinterpret_cast<float *>(w + g.states);
    const int64_t nchunks = (p->T + chunk - 1) / chunk;
    hipError_t e = launch_rotate(c, p->dtype, Q, qr, 1.f, st);
    if (e == hipSuccess) e = launch_rotate(c, p->dtype, K, kr, c.scale, st);
    if (e == hipSuccess) e = launch_generic_state(c, p->dtype, chunk, kr, V, state_in, state_out, cs, st);
    if (e == hipSuccess) {
        main_kernel_begin(st);
        e = launch_generic_output(c, p->dtype, chunk, qr, kr, V, O, cs,
                                  nchunks * p->dk * p->dv, (int64_t)p->dk * p->dv, st);
        main_kernel_end(st);
    }
    return hip_status(e, "generic chunkwise");
}

msr_status msr_recurrent_step(const msr_problem *p, const void *q, const void *k, const void *v,
                              void *o, float *state, void *hip_stream) {
    msr_status s = check_problem(p, true);
    if (s != MSR_OK) return s;
    if (p->B == 0) return MSR_OK;
    if (!q || !k || !v || !o || !state)
        return fail(MSR_ERR_INVALID_ARG, "q, k, v, o and state must be non-NULL");
    const void *ptrs[5] = {q, k, v, o, state};
    for (int i = 0; i < 5; ++i)
        if (!aligned16(ptrs[i])) return fail(MSR_ERR_INVALID_ARG, "pointer %d is not 16-byte aligned", i);
    if (o == q || o == k || o == v || o == (void *)state)
        return fail(MSR_ERR_INVALID_ARG, "o must not alias q, k, v or state");
    const MsrConst c = make_const(p, 1);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    main_kernel_begin(st);
    const hipError_t e = launch_decode(c, p->dtype, q, k, v, o, state, state, st);
    main_kernel_end(st);
    return hip_status(e, "decode step");
}

}  // extern "C"
