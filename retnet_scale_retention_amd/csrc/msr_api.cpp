// msr_api.cpp -- the C ABI of libmsr.so (declared in include/msr.h):
// argument validation, per-call constants, workspace carving and dispatch
// to the HIP kernels.  Validation completes before the first launch, so a
// non-OK status never leaves partial results behind.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "msr_internal.hpp"
#include "msr_chunk.hpp"
#include "msr_mfma.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
std::atomic<int> g_exchange{MSR_EXCHANGE_AUTO};

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
    if (p->flags & ~(uint32_t)(MSR_FLAG_NO_ROTATE | MSR_FLAG_NO_GROUPNORM | MSR_FLAG_DECAY_ROWNORM |
                               MSR_FLAG_SPLIT_SCORES | MSR_FLAG_FUSED))
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

// The general-purpose chunkwise path (any shape, either dtype, any chunk):
// rotation into fp32 copies, chunk-entry states, outputs.  ws holds
// generic_plan(p, MSR_FORM_CHUNKWISE, chunk).total bytes.
hipError_t generic_chunkwise(const msr_problem *p, int chunk, const void *Q, const void *K, const void *V, void *O,
                             const float *state_in, float *state_out, void *ws, hipStream_t st) {
    const MsrConst c = make_const(p, chunk);
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
        e = launch_generic_output(c, p->dtype, chunk, qr, kr, V, O, cs, nchunks * p->dk * p->dv,
                                  (int64_t)p->dk * p->dv, st);
        main_kernel_end(st);
    }
    return e;
}

// ---- backward pass ------------------------------------------------------------
// The retention-only sub-problems of the backward pass: fp32, no rotation, no
// GroupNorm, scale 1, dimensions d1 (queries and keys) and d2 (values).
msr_problem retention_problem(const msr_problem *p, int d1, int d2) {
    msr_problem r = *p;
    r.dk = d1;
    r.dv = d2;
    r.dtype = MSR_F32;
    r.theta = nullptr;
    r.scale = 1.f;
    r.pos0 = 0;
    r.pos_rows = nullptr;
    r.flags = MSR_FLAG_NO_ROTATE | MSR_FLAG_NO_GROUPNORM;
    return r;
}

// workspace: fp32 token-major tensors (N = B T H rows) and states, then the
// general path's own workspace for the largest of its four calls
struct BackPlan {
    size_t qf = 0, kf = 0, vf = 0, qr = 0, kr = 0, oraw = 0, g = 0, vrev = 0, grev = 0, qrrev = 0, krrev = 0,
           dq = 0, dkrev = 0, dvrev = 0, tmp = 0, s1 = 0, s2 = 0, s3 = 0, gws = 0, total = 0;
};

BackPlan back_plan(const msr_problem *p, int chunk) {
    BackPlan b;
    const size_t N = (size_t)p->B * p->T * p->H, dk = p->dk, dv = p->dv;
    const size_t st = round_up((size_t)p->B * p->H * dk * dv * sizeof(float));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += round_up(bytes);
        return o;
    };
    const bool copy = p->dtype != MSR_F32;  // fp32 inputs are used in place
    b.qf = copy ? take(N * dk * 4) : 0;
    b.kf = copy ? take(N * dk * 4) : 0;
    b.vf = copy ? take(N * dv * 4) : 0;
    b.qr = take(N * dk * 4);
    b.kr = take(N * dk * 4);
    b.oraw = take(N * dv * 4);
    b.g = take(N * dv * 4);
    b.vrev = take(N * dv * 4);
    b.grev = take(N * dv * 4);
    b.qrrev = take(N * dk * 4);
    b.krrev = take(N * dk * 4);
    b.dq = take(N * dk * 4);
    b.dkrev = take(N * dk * 4);
    b.dvrev = take(N * dv * 4);
    b.tmp = take(N * dk * 4);
    b.s1 = take(st);
    b.s2 = take(st);
    b.s3 = take(st);
    msr_problem a = retention_problem(p, p->dk, p->dv), t = retention_problem(p, p->dv, p->dk);
    const size_t g1 = generic_plan(&a, MSR_FORM_CHUNKWISE, chunk).total;
    const size_t g2 = generic_plan(&t, MSR_FORM_CHUNKWISE, chunk).total;
    b.gws = take(g1 > g2 ? g1 : g2);
    b.total = off;
    return b;
}

// The bf16 backward on the MFMA kernels.  The two products whose scores
// contract over d_v (queries G or V, keys V or G) take d_v in parts of at
// most 256 (the MFMA kernels' d_k range): the scores are sums over the
// contraction, so the parts' outputs add up.
constexpr int kMaxParts = 16;
int dv_parts(int dv, int *off, int *len) {
    int n = 0, o = 0;
    while (o < dv && n < kMaxParts) {
        const int r = dv - o, l = r >= 256 ? 256 : r >= 128 ? 128 : 64;
        off[n] = o;
        len[n] = l;
        o += l;
        ++n;
    }
    return o == dv ? n : -1;
}

msr_problem mfma_sub(const msr_problem *p, int d1, int d2) {
    msr_problem r = retention_problem(p, d1, d2);
    r.dtype = MSR_BF16;
    r.flags |= msr::kFlagNoWide;  // the 64-column chunk kernels are faster for these calls
    return r;
}

// The retention calls of the backward pass may use any chunk size (the forms
// agree for every b); 64 runs fastest on the MFMA path.
int backward_chunk(const msr_problem *p, int chunk) { return p->T % 64 == 0 ? 64 : chunk; }

bool mfma_backward_ok(const msr_problem *p, int chunk) {
    if (p->dtype != MSR_BF16 || p->dv % 64 != 0) return false;
    int off[kMaxParts], len[kMaxParts];
    const int n = dv_parts(p->dv, off, len);
    if (n < 1) return false;
    msr_problem c = mfma_sub(p, p->dk, p->dv);
    if (!mfma_supported(&c, MSR_FORM_CHUNKWISE, chunk)) return false;
    for (int i = 0; i < n; ++i) {
        msr_problem a = mfma_sub(p, len[i], p->dk);
        if (!mfma_supported(&a, MSR_FORM_CHUNKWISE, chunk)) return false;
    }
    return true;
}

struct BackPlanM {
    size_t oraw = 0, g = 0, qr = 0, kr = 0, ql = 0, kl = 0, qrrev = 0, grev = 0,
           part = 0, part2 = 0, acc = 0, s1 = 0, s2 = 0, s3 = 0, s4 = 0, mws = 0, total = 0;
};

BackPlanM back_plan_mfma(const msr_problem *p, int chunk) {
    BackPlanM b;
    const size_t N = (size_t)p->B * p->T * p->H, dk = p->dk, dv = p->dv;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += round_up(bytes);
        return o;
    };
    b.oraw = take(N * dv * 2);
    b.g = take(N * dv * 2);
    b.qr = take(N * dk * 2);
    b.kr = take(N * dk * 2);
    b.ql = take(N * dk * 2);
    b.kl = take(N * dk * 2);
    b.qrrev = take(N * dk * 2);
    b.grev = take(N * dv * 2);
    b.part = take(N * dk * 2);
    b.part2 = take(N * dk * 2);
    int poff[kMaxParts], plen[kMaxParts];
    b.acc = take(dv_parts(p->dv, poff, plen) > 2 ? N * dk * 4 : 0);  // fp32 sum of the parts beyond two
    const size_t sp = (size_t)p->B * p->H * 256 * dk * 4, sf = (size_t)p->B * p->H * dk * dv * 4;
    b.s1 = take(sp);
    b.s2 = take(sp);
    b.s3 = take(sf);
    b.s4 = take(sf);
    size_t m = mfma_workspace_bytes(p, MSR_FORM_CHUNKWISE, chunk);
    msr_problem c = mfma_sub(p, p->dk, p->dv);
    if (mfma_workspace_bytes(&c, MSR_FORM_CHUNKWISE, chunk) > m) m = mfma_workspace_bytes(&c, MSR_FORM_CHUNKWISE, chunk);
    for (int l = 64; l <= 256; l *= 2) {
        msr_problem a = mfma_sub(p, l, p->dk);
        const size_t x = mfma_workspace_bytes(&a, MSR_FORM_CHUNKWISE, chunk);
        if (x > m) m = x;
    }
    b.mws = take(m);
    b.total = off;
    return b;
}

// One retention call on the MFMA path (no rotation, no GroupNorm, scale 1).
// (Qlo, Klo: low parts of two-term bf16 splits of Q and K for the scores;
// ldqk: elements between rows of Q and K when they are column slices of
// wider rows, 0 for packed rows; revqk: Q, K (and Qlo, Klo) are read in
// reverse time order, V is taken as given)
hipError_t mfma_ret(const msr_problem *sub, int chunk, const void *Q, const void *K, const void *V, void *O,
                    const float *s_in, float *s_out, void *ws, hipStream_t st, const void *Qlo = nullptr,
                    const void *Klo = nullptr, int ldqk = 0, int revqk = 0) {
    MsrConst c = make_const(sub, chunk);
    c.ldqk = ldqk;
    c.revqk = revqk;
    return mfma_chunkwise(c, sub, chunk, Q, K, V, O, s_in, s_out, ws, st, Qlo, Klo);
}

hipError_t backward_mfma(const msr_problem *p, int chunk, const void *Q, const void *K, const void *V,
                         const float *state_in, const void *dO, const float *dstate_out, void *dQ, void *dK,
                         void *dV, float *dstate_in, void *ws, hipStream_t st) {
    const MsrConst c = make_const(p, chunk);
    const BackPlanM b = back_plan_mfma(p, chunk);
    char *w = static_cast<char *>(ws);
    auto P = [&](size_t o) { return static_cast<void *>(w + o); };
    auto F = [&](size_t o) { return reinterpret_cast<float *>(w + o); };
    const int dk = p->dk, dv = p->dv, B = p->B, T = p->T, H = p->H;
    const size_t N = (size_t)B * T * H;
    const int BF = MSR_BF16;
    int off[kMaxParts], len[kMaxParts];
    const int np = dv_parts(dv, off, len);
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t x) { if (e == hipSuccess) e = x; };
    const msr_problem pc = mfma_sub(p, dk, dv);
    // the rows of O are the pre-norm outputs times a per-row factor when the
    // decay is row-normalised: GroupNorm's input carries it, and so does G
    const bool rownorm = p->flags & MSR_FLAG_DECAY_ROWNORM;
    // 1. Q~ and K~ (scaled) as two-term bf16 splits hi + lo.  The
    //    intra-chunk score products q~_n . k~_m take hi.hi + lo.hi + hi.lo
    //    (in prep_kernel): a score much smaller than |q~||k~| loses its
    //    relative accuracy when q~ and k~ are rounded to bf16, and GroupNorm's
    //    backward amplifies that error on rows built from few tokens.
    //    Elsewhere Q~ and K~ enter as hi.
    ok(launch_rotate_tok(c, Q, BF, P(b.qr), BF, 1.f, 1.f, st, P(b.ql)));
    ok(launch_rotate_tok(c, K, BF, P(b.kr), BF, c.scale, 1.f, st, P(b.kl)));
    // 2. outputs before GroupNorm (bf16), then G = dL/dO_raw (bf16) by
    //    GroupNorm's backward
    const void *g = dO;
    if (!(p->flags & MSR_FLAG_NO_GROUPNORM)) {
        ok(mfma_ret(&pc, chunk, P(b.qr), P(b.kr), V, P(b.oraw), state_in, nullptr, P(b.mws), st, P(b.ql), P(b.kl)));
        if (rownorm) ok(launch_row_scale(c, dv, P(b.oraw), BF, P(b.oraw), BF, st));
        ok(launch_gn_backward(N, dv, c.eps, P(b.oraw), BF, dO, BF, P(b.g), BF, st));
        if (rownorm) ok(launch_row_scale(c, dv, P(b.g), BF, P(b.g), BF, st));
        g = P(b.g);
    } else if (rownorm) {
        ok(launch_row_scale(c, dv, dO, BF, P(b.g), BF, st));
        g = P(b.g);
    }
    // 3. dq~ = sum over the d_v parts of Ret(G_part, V_part, K~; S_in^T rows of the part);
    //    the parts are read in place as column slices (row stride d_v)
    auto col = [](const void *x, int c0) { return static_cast<const void *>(static_cast<const uint16_t *>(x) + c0); };
    //    The parts' results (bf16) are summed inside the inverse rotation:
    //    the last part from b.part, the others from b.part2 (two parts) or
    //    accumulated in fp32 in b.acc (more than two).
    auto part_out = [&](int i) { return P(i == np - 1 ? b.part : b.part2); };
    const void *part_sum = np == 1 ? P(b.part) : np == 2 ? P(b.part2) : P(b.acc);
    const int sum_dtype = np > 2 ? MSR_F32 : BF;
    const void *part_last = np > 1 ? P(b.part) : nullptr;
    for (int i = 0; i < np && e == hipSuccess; ++i) {
        const msr_problem a = mfma_sub(p, len[i], dk);
        float *sinT = state_in ? F(b.s1) : nullptr;
        if (state_in) ok(launch_state_op(c, dk, dv, state_in, sinT, 1, 0.f, off[i], len[i], st));
        ok(mfma_ret(&a, chunk, col(g, off[i]), col(V, off[i]), P(b.kr), part_out(i), sinT, nullptr, P(b.mws), st,
                    nullptr, nullptr, dv));
        if (np > 2 && i < np - 1) ok(launch_accumulate(N * dk, P(b.part2), BF, F(b.acc), i == 0, st));
    }
    ok(launch_rotate_tok(c, part_sum, sum_dtype, dQ, BF, 1.f, -1.f, st, nullptr, 0, part_last));
    // 4. dk~ (backward in time) = sum over parts of Ret(V_part, G_part, Q~; dS_out^T / gamma rows);
    //    the prep kernel reads V_part and G_part in reverse time order in
    //    place, the value operand Q~ is a reversed copy
    ok(launch_slice(B, T, H, dk, 0, dk, 1, P(b.qr), BF, P(b.qrrev), BF, st));
    for (int i = 0; i < np && e == hipSuccess; ++i) {
        const msr_problem a = mfma_sub(p, len[i], dk);
        float *dsoT = dstate_out ? F(b.s2) : nullptr;
        if (dstate_out) ok(launch_state_op(c, dk, dv, dstate_out, dsoT, 1, -1.f, off[i], len[i], st));
        ok(mfma_ret(&a, chunk, col(V, off[i]), col(g, off[i]), P(b.qrrev), part_out(i), dsoT, nullptr, P(b.mws),
                    st, nullptr, nullptr, dv, 1));
        if (np > 2 && i < np - 1) ok(launch_accumulate(N * dk, P(b.part2), BF, F(b.acc), i == 0, st));
    }
    ok(launch_rotate_tok(c, part_sum, sum_dtype, dK, BF, c.scale, -1.f, st, nullptr, 1, part_last));
    // 5. dV (backward in time) = Ret(K~, Q~, G; dS_out / gamma), its scores
    //    split as in 1.; its outgoing state times gamma is dS_in
    //    (K~, Q~ and their low parts read reversed in place, G as a reversed copy)
    ok(launch_slice(B, T, H, dv, 0, dv, 1, g, BF, P(b.grev), BF, st));
    float *dso = dstate_out ? F(b.s3) : nullptr, *sc = dstate_in ? F(b.s4) : nullptr;
    if (dstate_out) ok(launch_state_op(c, dk, dv, dstate_out, dso, 0, -1.f, 0, dv, st));
    ok(mfma_ret(&pc, chunk, P(b.kr), P(b.qr), P(b.grev), P(b.oraw), dso, sc, P(b.mws), st, P(b.kl), P(b.ql), 0,
                1));
    ok(launch_slice(B, T, H, dv, 0, dv, 1, P(b.oraw), BF, dV, BF, st));
    if (dstate_in) ok(launch_state_op(c, dk, dv, sc, dstate_in, 0, 1.f, 0, dv, st));
    return e;
}

// ---- split scores (MSR_FLAG_SPLIT_SCORES) ----------------------------------

// Heads whose decay is below this take the split scores by default.  Under
// strong decay a row's output comes from a few recent tokens; when their
// scores are small against |q~||k~|, bf16 rounding of q~ and k~ costs the
// scores their relative accuracy, and GroupNorm amplifies that on the row.
// A CPU emulation that rounds only the rotated q~, k~ to bf16 (d_k 64 and
// 256, T = 256, four seeds) puts the plain path at 7.7e-3 for gamma = 0.9,
// 1.3e-2 at 0.8, 1.6e-2 at 0.75 and 3.3e-2 at 0.5, against the 2e-2 bf16
// tolerance; the threshold keeps the plain path where it has margin.
constexpr float kSplitGamma = 0.9f;

bool strong_decay(const msr_problem *p) {
    for (int h = 0; h < p->H; ++h)
        if (p->gamma[h] < kSplitGamma) return true;
    return false;
}

bool split_scores(const msr_problem *p, int chunk) {
    return ((p->flags & MSR_FLAG_SPLIT_SCORES) || strong_decay(p)) && p->T > MSR_DECODE_MAX_T &&
           mfma_supported(p, MSR_FORM_CHUNKWISE, chunk);
}

// The parallel form under strong decay runs as the chunkwise form with split
// scores (the forms are equal, state included); the chunk size is the first
// of 64, 128, 256 the matrix-core path takes for this T, 0 if none.
int parallel_split_chunk(const msr_problem *p) {
    if (!strong_decay(p) || p->T <= MSR_DECODE_MAX_T) return 0;
    for (int b = 64; b <= 256; b *= 2)
        if (split_scores(p, b)) return b;
    return 0;
}

// workspace in front of the chunkwise workspace: Q~ and K~ (scaled) as hi, lo bf16 pairs
struct SplitPlan {
    size_t qh = 0, ql = 0, kh = 0, kl = 0, total = 0;
};

SplitPlan split_plan(const msr_problem *p) {
    SplitPlan b;
    const size_t t = round_up((size_t)p->B * p->T * p->H * p->dk * 2);
    b.qh = 0;
    b.ql = t;
    b.kh = 2 * t;
    b.kl = 3 * t;
    b.total = 4 * t;
    return b;
}

hipError_t chunkwise_split(const msr_problem *p, int chunk, const void *Q, const void *K, const void *V, void *O,
                           const float *s_in, float *s_out, void *ws, hipStream_t st) {
    const MsrConst c = make_const(p, chunk);
    const SplitPlan b = split_plan(p);
    char *w = static_cast<char *>(ws);
    hipError_t e = launch_rotate_tok(c, Q, MSR_BF16, w + b.qh, MSR_BF16, 1.f, 1.f, st, w + b.ql);
    if (e == hipSuccess) e = launch_rotate_tok(c, K, MSR_BF16, w + b.kh, MSR_BF16, c.scale, 1.f, st, w + b.kl);
    if (e != hipSuccess) return e;
    msr_problem sub = *p;  // rotated and scaled already; positions stay for the row factors
    sub.flags |= MSR_FLAG_NO_ROTATE;
    sub.scale = 1.f;
    return mfma_chunkwise(make_const(&sub, chunk), &sub, chunk, w + b.qh, w + b.kh, V, O, s_in, s_out, w + b.total,
                          st, w + b.ql, w + b.kl);
}

// ---- Q/K/V projections -------------------------------------------------

// the chunkwise problem over projected inputs: rotation and scale already applied
msr_problem qkv_sub(const msr_problem *p) {
    msr_problem r = *p;
    r.flags |= MSR_FLAG_NO_ROTATE;
    r.scale = 1.f;
    return r;
}

struct QkvPlan {
    size_t q = 0, k = 0, v = 0, total = 0;
};

QkvPlan qkv_plan(const msr_problem *p) {
    QkvPlan b;
    const size_t M = (size_t)p->B * p->T;
    b.q = 0;
    b.k = round_up(M * p->H * p->dk * 2);
    b.v = b.k + round_up(M * p->H * p->dk * 2);
    b.total = b.v + round_up(M * p->H * p->dv * 2);
    return b;
}

msr_status check_qkv(const msr_problem *p, int d_model, const void *X, const void *Wq, const void *Wk,
                     const void *Wv) {
    msr_status s = check_problem(p, false);
    if (s != MSR_OK) return s;
    if (p->dtype != MSR_BF16) return fail(MSR_ERR_UNSUPPORTED, "the projections take bf16 only");
    if (d_model <= 0 || d_model % 64 != 0)
        return fail(MSR_ERR_SHAPE, "d_model=%d must be a positive multiple of 64", d_model);
    if ((p->H * p->dk) % 4 != 0) return fail(MSR_ERR_SHAPE, "H*dk=%d must be a multiple of 4", p->H * p->dk);
    const bool any = (size_t)p->B * p->T > 0;
    const void *in[4] = {X, Wq, Wk, Wv};
    const char *names[4] = {"X", "Wq", "Wk", "Wv"};
    for (int i = 0; i < 4; ++i) {
        if (any && !in[i]) return fail(MSR_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (in[i] && !aligned16(in[i])) return fail(MSR_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    return MSR_OK;
}

}  // namespace

void main_kernel_begin(hipStream_t st) {
    if (g_ev_start) (void)hipEventRecord(g_ev_start, st);
}

void main_kernel_end(hipStream_t st) {
    if (g_ev_stop) (void)hipEventRecord(g_ev_stop, st);
}

int exchange_mode() { return g_exchange.load(std::memory_order_relaxed); }

hipEvent_t main_event_start() { return g_ev_start; }
hipEvent_t main_event_stop() { return g_ev_stop; }

extern "C" {

int msr_abi_version(void) { return MSR_ABI_VERSION; }

void msr_set_kernel_events(void *start, void *stop) {
    g_ev_start = static_cast<hipEvent_t>(start);
    g_ev_stop = static_cast<hipEvent_t>(stop);
}

msr_status msr_set_exchange(int32_t mode) {
    if (mode != MSR_EXCHANGE_AUTO && mode != MSR_EXCHANGE_OFF && mode != MSR_EXCHANGE_NO_WAIT)
        return fail(MSR_ERR_INVALID_ARG, "exchange mode %d is not one of 0, 1, 2", (int)mode);
    g_exchange.store(mode, std::memory_order_relaxed);
    return MSR_OK;
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
    if (form == MSR_FORM_BACKWARD) {
        if (chunk < 1) return fail(MSR_ERR_SHAPE, "chunk=%d must be >= 1", chunk);
        if (p->dv > MSR_MAX_DK)
            return fail(MSR_ERR_UNSUPPORTED, "the backward pass needs dv <= %d (dv=%d)", MSR_MAX_DK, p->dv);
        const int bc = backward_chunk(p, chunk);
        *bytes = mfma_backward_ok(p, bc) ? back_plan_mfma(p, bc).total : back_plan(p, chunk).total;
        return MSR_OK;
    }
    if (form == MSR_FORM_QKV_CHUNKWISE) {
        if (chunk < 1) return fail(MSR_ERR_SHAPE, "chunk=%d must be >= 1", chunk);
        const msr_problem sub = qkv_sub(p);
        size_t inner = 0;
        if ((s = msr_workspace_size(&sub, MSR_FORM_CHUNKWISE, chunk, &inner)) != MSR_OK) return s;
        *bytes = qkv_plan(p).total + inner;
        return MSR_OK;
    }
    if (form == MSR_FORM_CHUNKWISE) {
        if (chunk < 1) return fail(MSR_ERR_SHAPE, "chunk=%d must be >= 1", chunk);
    } else if (form != MSR_FORM_PARALLEL) {
        return fail(MSR_ERR_INVALID_ARG, "unknown form %d", form);
    }
    size_t need = generic_plan(p, form, chunk).total;
    size_t mf = mfma_workspace_bytes(p, form, chunk);
    if (form == MSR_FORM_CHUNKWISE && split_scores(p, chunk))
        mf = split_plan(p).total + mfma_workspace_bytes(p, form, chunk, true);
    if (form == MSR_FORM_PARALLEL) {
        const int b = parallel_split_chunk(p);
        if (b) mf = split_plan(p).total + mfma_workspace_bytes(p, MSR_FORM_CHUNKWISE, b, true);
    }
    if (mf > need) need = mf;
    *bytes = need;
    return MSR_OK;
}

size_t msr_workspace_bytes(const msr_problem *p, int32_t form, int32_t chunk) {
    size_t n = 0;
    return msr_workspace_size(p, form, chunk, &n) == MSR_OK ? n : 0;
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

    if (const int b = parallel_split_chunk(p))
        return hip_status(chunkwise_split(p, b, Q, K, V, O, state_in, state_out, ws, st), "split parallel");
    if (mfma_supported(p, MSR_FORM_PARALLEL, p->T))
        return hip_status(mfma_parallel(c, p, Q, K, V, O, state_in, state_out, ws, st), "mfma parallel");
    if (p->T <= MSR_DECODE_MAX_T) {  // a few tokens: the recurrence, one pass over the state
        const hipError_t e = launch_decode(c, p->dtype, Q, K, V, O, state_in, state_out, st);
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

    if (split_scores(p, chunk))
        return hip_status(chunkwise_split(p, chunk, Q, K, V, O, state_in, state_out, ws, st), "split chunkwise");
    if (mfma_supported(p, MSR_FORM_CHUNKWISE, chunk))
        return hip_status(mfma_chunkwise(c, p, chunk, Q, K, V, O, state_in, state_out, ws, st),
                          "mfma chunkwise");
    if (p->T <= MSR_DECODE_MAX_T) {  // a few tokens: one pass over the state (the result is independent of b)
        const hipError_t e = launch_decode(c, p->dtype, Q, K, V, O, state_in, state_out, st);
        return hip_status(e, "short chunkwise");
    }

    return hip_status(generic_chunkwise(p, chunk, Q, K, V, O, state_in, state_out, ws, st), "generic chunkwise");
}

msr_status msr_chunkwise_noalloc(const msr_problem *p, int32_t chunk, const void *Q, const void *K,
                                 const void *V, void *O, const float *state_in, float *state_out,
                                 void *hip_stream) {
    msr_status s = check_problem(p, false);
    if (s != MSR_OK) return s;
    if ((s = check_tensors(p, Q, K, V, O, state_in, state_out)) != MSR_OK) return s;
    size_t need = 0;
    if ((s = msr_workspace_size(p, MSR_FORM_CHUNKWISE, chunk, &need)) != MSR_OK) return s;
    if (need > MSR_STATIC_SCRATCH_BYTES)
        return fail(MSR_ERR_WORKSPACE,
                    "this call needs %zu bytes of scratch, more than the %zu of the fixed array "
                    "msr_chunkwise_noalloc uses (call msr_chunkwise with a workspace instead)",
                    need, MSR_STATIC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0 && (size_t)p->B * p->T > 0) {
        const hipError_t e = static_scratch(&ws);
        if (e != hipSuccess) return hip_status(e, "scratch address");
    }
    return msr_chunkwise(p, chunk, Q, K, V, O, state_in, state_out, ws, ws ? MSR_STATIC_SCRATCH_BYTES : 0,
                         hip_stream);
}

msr_status msr_qkv_projection(const msr_problem *p, int32_t d_model, const void *X, const void *Wq,
                              const void *Wk, const void *Wv, void *Q, void *K, void *V, void *hip_stream) {
    msr_status s = check_qkv(p, d_model, X, Wq, Wk, Wv);
    if (s != MSR_OK) return s;
    const size_t M = (size_t)p->B * p->T;
    if (M == 0) return MSR_OK;
    if (M > (size_t)INT32_MAX) return fail(MSR_ERR_SHAPE, "B*T is too large");
    const void *outs[3] = {Q, K, V};
    const char *on[3] = {"Q", "K", "V"};
    const void *ins[4] = {X, Wq, Wk, Wv};
    for (int i = 0; i < 3; ++i) {
        if (!outs[i]) return fail(MSR_ERR_INVALID_ARG, "%s is NULL", on[i]);
        if (!aligned16(outs[i])) return fail(MSR_ERR_INVALID_ARG, "%s is not 16-byte aligned", on[i]);
        for (int j = 0; j < 4; ++j)
            if (outs[i] == ins[j]) return fail(MSR_ERR_INVALID_ARG, "%s must not alias an input", on[i]);
        for (int j = 0; j < i; ++j)
            if (outs[i] == outs[j]) return fail(MSR_ERR_INVALID_ARG, "%s must not alias %s", on[i], on[j]);
    }
    const MsrConst c = make_const(p, p->T);
    const void *W[3] = {Wq, Wk, Wv};
    void *Y[3] = {Q, K, V};
    const int n[3] = {p->H * p->dk, p->H * p->dk, p->H * p->dv};
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    return hip_status(launch_proj(c, (int)M, d_model, X, W, Y, n, !(p->flags & MSR_FLAG_NO_ROTATE), st),
                      "qkv projection");
}

msr_status msr_qkv_chunkwise(const msr_problem *p, int32_t chunk, int32_t d_model, const void *X,
                             const void *Wq, const void *Wk, const void *Wv, void *O, const float *state_in,
                             float *state_out, void *ws, size_t ws_bytes, void *hip_stream) {
    msr_status s = check_qkv(p, d_model, X, Wq, Wk, Wv);
    if (s != MSR_OK) return s;
    size_t need = 0;
    if ((s = msr_workspace_size(p, MSR_FORM_QKV_CHUNKWISE, chunk, &need)) != MSR_OK) return s;
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(MSR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
    if (ws && !aligned16(ws)) return fail(MSR_ERR_INVALID_ARG, "ws is not 16-byte aligned");
    const QkvPlan b = qkv_plan(p);
    char *w = static_cast<char *>(ws);
    const msr_problem sub = qkv_sub(p);
    // validate the retention call before anything runs
    if ((s = check_tensors(&sub, w + b.q, w + b.k, w + b.v, O, state_in, state_out)) != MSR_OK) return s;
    if ((s = msr_qkv_projection(p, d_model, X, Wq, Wk, Wv, w + b.q, w + b.k, w + b.v, hip_stream)) != MSR_OK)
        return s;
    return msr_chunkwise(&sub, chunk, w + b.q, w + b.k, w + b.v, O, state_in, state_out, w + b.total,
                         ws_bytes - b.total, hip_stream);
}

msr_status msr_chunkwise_backward(const msr_problem *p, int32_t chunk, const void *Q, const void *K,
                                  const void *V, const float *state_in, const void *dO,
                                  const float *dstate_out, void *dQ, void *dK, void *dV, float *dstate_in,
                                  void *ws, size_t ws_bytes, void *hip_stream) {
    msr_status s = check_problem(p, false);
    if (s != MSR_OK) return s;
    size_t need = 0;
    if ((s = msr_workspace_size(p, MSR_FORM_BACKWARD, chunk, &need)) != MSR_OK) return s;
    const bool any = (size_t)p->B * p->T > 0;
    if (any && (!Q || !K || !V || !dO || !dQ || !dK || !dV))
        return fail(MSR_ERR_INVALID_ARG, "Q, K, V, dO, dQ, dK and dV must be non-NULL");
    const void *ptrs[10] = {Q, K, V, state_in, dO, dstate_out, dQ, dK, dV, dstate_in};
    const char *names[10] = {"Q", "K", "V", "state_in", "dO", "dstate_out", "dQ", "dK", "dV", "dstate_in"};
    for (int i = 0; i < 10; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(MSR_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    for (int i = 6; i < 10; ++i)
        for (int j = 0; j < 10; ++j)
            if (i != j && ptrs[i] && ptrs[i] == ptrs[j])
                return fail(MSR_ERR_INVALID_ARG, "%s must not alias %s", names[i], names[j]);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(MSR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
    if (ws && !aligned16(ws)) return fail(MSR_ERR_INVALID_ARG, "ws is not 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const MsrConst c = make_const(p, chunk);
    if (p->B == 0) return MSR_OK;
    const int dk = p->dk, dv = p->dv, B = p->B, T = p->T, H = p->H;
    if (T == 0) {  // state_out = state_in: dstate_in = dstate_out
        if (!dstate_in) return MSR_OK;
        return hip_status(launch_state_op(c, dk, dv, dstate_out, dstate_in, 0, 0.f, 0, dv, st), "backward");
    }
    if (mfma_backward_ok(p, backward_chunk(p, chunk)))
        return hip_status(backward_mfma(p, backward_chunk(p, chunk), Q, K, V, state_in, dO, dstate_out, dQ, dK, dV,
                                        dstate_in, ws, st),
                          "backward (mfma)");
    const BackPlan b = back_plan(p, chunk);
    char *w = static_cast<char *>(ws);
    auto F = [&](size_t off) { return reinterpret_cast<float *>(w + off); };
    const size_t N = (size_t)B * T * H;
    const bool copy = p->dtype != MSR_F32;
    const float *qf = copy ? F(b.qf) : static_cast<const float *>(Q);
    const float *kf = copy ? F(b.kf) : static_cast<const float *>(K);
    const float *vf = copy ? F(b.vf) : static_cast<const float *>(V);
    float *qr = F(b.qr), *kr = F(b.kr), *oraw = F(b.oraw), *g = F(b.g), *gws = F(b.gws);
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t x) { if (e == hipSuccess) e = x; };
    if (copy) {
        ok(launch_to_f32(p->dtype, N * dk, Q, F(b.qf), st));
        ok(launch_to_f32(p->dtype, N * dk, K, F(b.kf), st));
        ok(launch_to_f32(p->dtype, N * dv, V, F(b.vf), st));
    }
    // 1. forward outputs before GroupNorm, and G = dL/dO_raw
    msr_problem pf = *p;
    pf.dtype = MSR_F32;
    pf.flags |= MSR_FLAG_NO_GROUPNORM;
    ok(generic_chunkwise(&pf, chunk, qf, kf, vf, oraw, state_in, nullptr, gws, st));
    // (with row-normalised decay, oraw already carries the row factor, and G
    // takes it once more: O = GN(f O_raw))
    if (!(p->flags & MSR_FLAG_NO_GROUPNORM))
        ok(launch_gn_backward(N, dv, c.eps, oraw, MSR_F32, dO, p->dtype, g, MSR_F32, st));
    else
        ok(launch_to_f32(p->dtype, N * dv, dO, g, st));
    if (p->flags & MSR_FLAG_DECAY_ROWNORM) ok(launch_row_scale(c, dv, g, MSR_F32, g, MSR_F32, st));
    // 2. rotated (and scaled) Q~, K~, token-major fp32
    ok(launch_rotate_tok(c, qf, MSR_F32, qr, MSR_F32, 1.f, 1.f, st));
    ok(launch_rotate_tok(c, kf, MSR_F32, kr, MSR_F32, c.scale, 1.f, st));
    // 3. dq~ = Ret(G, V, K~; S_in^T)
    const msr_problem pa = retention_problem(p, dv, dk), pc = retention_problem(p, dk, dv);
    float *sinT = state_in ? F(b.s1) : nullptr;
    if (state_in) ok(launch_state_op(c, dk, dv, state_in, sinT, 1, 0.f, 0, dv, st));
    ok(generic_chunkwise(&pa, chunk, g, vf, kr, F(b.dq), sinT, nullptr, gws, st));
    // 4. the same tensors backward in time
    ok(launch_slice(B, T, H, dv, 0, dv, 1, vf, MSR_F32, F(b.vrev), MSR_F32, st));
    ok(launch_slice(B, T, H, dv, 0, dv, 1, g, MSR_F32, F(b.grev), MSR_F32, st));
    ok(launch_slice(B, T, H, dk, 0, dk, 1, qr, MSR_F32, F(b.qrrev), MSR_F32, st));
    ok(launch_slice(B, T, H, dk, 0, dk, 1, kr, MSR_F32, F(b.krrev), MSR_F32, st));
    // 5. dk~ (reversed) = Ret(V, G, Q~; dS_out^T / gamma)
    float *dsoT = dstate_out ? F(b.s2) : nullptr, *dso = dstate_out ? F(b.s3) : nullptr;
    if (dstate_out) {
        ok(launch_state_op(c, dk, dv, dstate_out, dsoT, 1, -1.f, 0, dv, st));
        ok(launch_state_op(c, dk, dv, dstate_out, dso, 0, -1.f, 0, dv, st));
    }
    ok(generic_chunkwise(&pa, chunk, F(b.vrev), F(b.grev), F(b.qrrev), F(b.dkrev), dsoT, nullptr, gws, st));
    // 6. dV (reversed) = Ret(K~, Q~, G; dS_out / gamma), whose outgoing state
    //    times gamma is dS_in (s1 is free again: the first call has run)
    float *sc = dstate_in ? F(b.s1) : nullptr;
    ok(generic_chunkwise(&pc, chunk, F(b.krrev), F(b.qrrev), F(b.grev), F(b.dvrev), dso, sc, gws, st));
    if (dstate_in) ok(launch_state_op(c, dk, dv, sc, dstate_in, 0, 1.f, 0, dv, st));
    // 7. back through the rotation and the scale, into the caller's dtype
    ok(launch_rotate_tok(c, F(b.dq), MSR_F32, dQ, p->dtype, 1.f, -1.f, st));
    ok(launch_slice(B, T, H, dk, 0, dk, 1, F(b.dkrev), MSR_F32, F(b.tmp), MSR_F32, st));
    ok(launch_rotate_tok(c, F(b.tmp), MSR_F32, dK, p->dtype, c.scale, -1.f, st));
    ok(launch_slice(B, T, H, dv, 0, dv, 1, F(b.dvrev), MSR_F32, dV, p->dtype, st));
    return hip_status(e, "backward");
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
    // (launch_decode attaches the kernel events to the step kernel itself)
    const hipError_t e = launch_decode(c, p->dtype, q, k, v, o, state, state, st);
    return hip_status(e, "decode step");
}

}  // extern "C"
