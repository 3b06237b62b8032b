// ttt_host.cpp -- the C ABI of libttt: argument checks, the split of a call
// into token-by-token and whole-mini-batch pieces, kernel launches.
//
// A call over L tokens starting at absolute position `offset`
// ("TTTBase.forward": whole mini-batches first, the remainder after it with
// the carried state; "TTTLinear.ttt": dual form for whole mini-batches, primal
// form when the gradient must be kept for a later call):
//   head : tokens up to the next multiple of K (completes an open mini-batch),
//   body : whole mini-batches, dual form on MFMA (K = 16),
//   tail : the last L' < K tokens, left open in the state.
// The three pieces are enqueued in order on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "launch.hpp"
#include "post_proj.hpp"
#include "ttt.h"

using namespace ttt;

namespace {

thread_local std::string g_last_error;

ttt_status fail(ttt_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

ttt_status ok() {
    g_last_error.clear();
    return TTT_OK;
}

size_t dtype_size(int32_t dt) { return dt == TTT_BF16 ? 2 : 4; }
bool dtype_valid(int32_t dt) { return dt == TTT_F32 || dt == TTT_BF16; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range tensor_range(const void *p, int64_t sB, int64_t sH, int64_t sL, int B, int H, int L, int D, size_t es) {
    const uintptr_t base = reinterpret_cast<uintptr_t>(p);
    const int64_t last = (int64_t)(B - 1) * sB + (int64_t)(H - 1) * sH + (int64_t)(L - 1) * sL + D;
    return Range{base, base + (uintptr_t)last * es};
}
Range flat_range(const void *p, int64_t n, size_t es) {
    const uintptr_t base = reinterpret_cast<uintptr_t>(p);
    return Range{base, base + (uintptr_t)n * es};
}

// Checks one activation descriptor.  `out` additionally needs a layout in
// which distinct (b, h, t) rows never share memory.
ttt_status check_tensor(const char *name, const void *p, int64_t sB, int64_t sH, int64_t sL, int B, int H, int L,
                        int D, size_t es, bool out) {
    if (!p) return fail(TTT_ERR_NULL, "%s is NULL", name);
    if (sB < 0 || sH < 0 || sL < 0) return fail(TTT_ERR_ALIGN, "%s has a negative stride", name);
    if (!aligned16(p)) return fail(TTT_ERR_ALIGN, "%s is not 16-byte aligned", name);
    if ((sB * (int64_t)es) % 16 || (sH * (int64_t)es) % 16 || (sL * (int64_t)es) % 16)
        return fail(TTT_ERR_ALIGN, "%s strides (%lld, %lld, %lld) are not multiples of 16 bytes", name, (long long)sB,
                    (long long)sH, (long long)sL);
    if (out) {
        // sort the (stride, extent) pairs of the non-trivial dims; each stride
        // must clear the span of the smaller ones
        std::vector<std::pair<int64_t, int64_t>> dims;
        if (B > 1) dims.push_back({sB, B});
        if (H > 1) dims.push_back({sH, H});
        if (L > 1) dims.push_back({sL, L});
        std::sort(dims.begin(), dims.end());
        int64_t span = D;
        for (auto &d : dims) {
            if (d.first < span) return fail(TTT_ERR_ALIAS, "%s has overlapping rows (stride %lld < %lld)", name,
                                            (long long)d.first, (long long)span);
            span = d.first * d.second;
        }
    }
    return TTT_OK;
}

ttt_status check_common(int32_t B, int32_t H, int32_t D, int32_t K, int32_t in_dt, int32_t out_dt, float eps,
                        float rope_base, int32_t rope) {
    if (B < 1 || H < 1) return fail(TTT_ERR_SHAPE, "B=%d, H=%d must be >= 1", B, H);
    if ((int64_t)B * H > (int64_t)INT32_MAX / 2) return fail(TTT_ERR_SHAPE, "B*H too large");
    if (D != 64) return fail(TTT_ERR_SHAPE, "head_dim D=%d unsupported (must be 64)", D);
    if (K < 1 || K > 16) return fail(TTT_ERR_SHAPE, "mini_batch_size K=%d outside 1..16", K);
    if (!dtype_valid(in_dt) || !dtype_valid(out_dt))
        return fail(TTT_ERR_DTYPE, "unknown dtype (in=%d, out=%d)", in_dt, out_dt);
    if (!(eps > 0.f)) return fail(TTT_ERR_SHAPE, "ln_eps must be > 0");
    if (rope != 0 && rope != 1) return fail(TTT_ERR_SHAPE, "rope must be 0 or 1");
    if (rope && !(rope_base > 1.f)) return fail(TTT_ERR_SHAPE, "rope_base must be > 1");
    return TTT_OK;
}

struct Act {
    ttt_tensor XQ, XK, XV, out;
    ttt_eta eta;
    const float *ln_w, *ln_b;
};

// Checks everything shared by the linear and MLP calls.  `state_ranges` are
// the device ranges of the state, which `out` must not overlap.
ttt_status check_acts(const Act &x, int B, int H, int L, int D, int K, int32_t in_dt, int32_t out_dt,
                      const std::vector<Range> &state_ranges) {
    const size_t ei = dtype_size(in_dt), eo = dtype_size(out_dt);
    ttt_status s;
    if ((s = check_tensor("XQ", x.XQ.data, x.XQ.sB, x.XQ.sH, x.XQ.sL, B, H, L, D, ei, false))) return s;
    if ((s = check_tensor("XK", x.XK.data, x.XK.sB, x.XK.sH, x.XK.sL, B, H, L, D, ei, false))) return s;
    if ((s = check_tensor("XV", x.XV.data, x.XV.sB, x.XV.sH, x.XV.sL, B, H, L, D, ei, false))) return s;
    if ((s = check_tensor("out", x.out.data, x.out.sB, x.out.sH, x.out.sL, B, H, L, D, eo, true))) return s;
    if (!x.eta.data) return fail(TTT_ERR_NULL, "eta is NULL");
    if (x.eta.sB < 0 || x.eta.sH < 0) return fail(TTT_ERR_ALIGN, "eta has a negative stride");
    if (!x.ln_w || !x.ln_b) return fail(TTT_ERR_NULL, "ln_w / ln_b is NULL");
    if (x.eta.token_eta && !aligned16(x.eta.token_eta)) return fail(TTT_ERR_ALIGN, "token_eta must be 16-byte aligned");
    const Range ro = tensor_range(x.out.data, x.out.sB, x.out.sH, x.out.sL, B, H, L, D, eo);
    const Range rin[] = {tensor_range(x.XQ.data, x.XQ.sB, x.XQ.sH, x.XQ.sL, B, H, L, D, ei),
                         tensor_range(x.XK.data, x.XK.sB, x.XK.sH, x.XK.sL, B, H, L, D, ei),
                         tensor_range(x.XV.data, x.XV.sB, x.XV.sH, x.XV.sL, B, H, L, D, ei),
                         tensor_range(x.eta.data, x.eta.sB, x.eta.sH, 1, B, H, L, 1, 4),
                         flat_range(x.ln_w, (int64_t)H * D, 4), flat_range(x.ln_b, (int64_t)H * D, 4),
                         flat_range(x.eta.token_eta, x.eta.token_eta ? K : 0, 4)};
    for (const Range &r : rin)
        if (overlap(ro, r)) return fail(TTT_ERR_ALIAS, "out overlaps an input");
    for (const Range &r : state_ranges) {
        if (overlap(ro, r)) return fail(TTT_ERR_ALIAS, "out overlaps the state");
        // the kernels write the state while they read the inputs
        for (const Range &i : rin)
            if (overlap(i, r)) return fail(TTT_ERR_ALIAS, "an input overlaps the state");
    }
    return TTT_OK;
}

ttt_status check_linear_state(const ttt_linear_cfg *cfg, const ttt_linear_state *st, std::vector<Range> &ranges,
                              bool check_offset = true) {
    if (!st) return fail(TTT_ERR_NULL, "state is NULL");
    if (!st->W || !st->b || !st->W_grad || !st->b_grad) return fail(TTT_ERR_NULL, "state buffer is NULL");
    if (!aligned16(st->W) || !aligned16(st->b) || !aligned16(st->W_grad) || !aligned16(st->b_grad))
        return fail(TTT_ERR_ALIGN, "state buffers must be 16-byte aligned");
    if (check_offset && st->offset < 0) return fail(TTT_ERR_STATE, "state offset %lld < 0", (long long)st->offset);
    const int64_t n = (int64_t)cfg->B * cfg->H;
    ranges = {flat_range(st->W, n * cfg->D * cfg->D, 4), flat_range(st->b, n * cfg->D, 4),
              flat_range(st->W_grad, n * cfg->D * cfg->D, 4), flat_range(st->b_grad, n * cfg->D, 4)};
    for (size_t i = 0; i < ranges.size(); ++i)
        for (size_t j = i + 1; j < ranges.size(); ++j)
            if (overlap(ranges[i], ranges[j])) return fail(TTT_ERR_ALIAS, "state buffers overlap");
    return TTT_OK;
}

ttt_status check_mlp_cfg(const ttt_mlp_cfg *cfg) {
    if (!cfg) return fail(TTT_ERR_NULL, "cfg is NULL");
    ttt_status s;
    if ((s = check_common(cfg->B, cfg->H, cfg->D, cfg->K, cfg->in_dtype, cfg->out_dtype, cfg->ln_eps,
                          cfg->rope_base, cfg->rope)))
        return s;
    if (cfg->F != 256) return fail(TTT_ERR_SHAPE, "MLP hidden width F=%d unsupported (must be 256)", cfg->F);
    if (cfg->grad_layout != TTT_GRAD_DENSE && cfg->grad_layout != TTT_GRAD_ROWS)
        return fail(TTT_ERR_UNSUPPORTED, "unknown grad_layout %d", (int)cfg->grad_layout);
    return TTT_OK;
}

ttt_status check_mlp_state(const ttt_mlp_cfg *cfg, const ttt_mlp_state *st, std::vector<Range> &ranges,
                           bool check_offset) {
    if (!st) return fail(TTT_ERR_NULL, "state is NULL");
    float *const p[8] = {st->W1, st->b1, st->W2, st->b2, st->W1_grad, st->b1_grad, st->W2_grad, st->b2_grad};
    for (float *q : p) {
        if (!q) return fail(TTT_ERR_NULL, "state buffer is NULL");
        if (!aligned16(q)) return fail(TTT_ERR_ALIGN, "state buffers must be 16-byte aligned");
    }
    if (check_offset && st->offset < 0) return fail(TTT_ERR_STATE, "state offset %lld < 0", (long long)st->offset);
    const int64_t n = (int64_t)cfg->B * cfg->H, D = cfg->D, F = cfg->F;
    const int64_t sz[8] = {D * F, F, F * D, D, D * F, F, F * D, D};
    ranges.clear();
    for (int i = 0; i < 8; ++i) ranges.push_back(flat_range(p[i], n * sz[i], 4));
    for (size_t i = 0; i < ranges.size(); ++i)
        for (size_t j = i + 1; j < ranges.size(); ++j)
            if (overlap(ranges[i], ranges[j])) return fail(TTT_ERR_ALIAS, "state buffers overlap");
    return TTT_OK;
}

LinearArgs linear_args(const ttt_linear_cfg *cfg, const Act &x, ttt_linear_state *st) {
    LinearArgs a{};
    a.q = TDesc{x.XQ.data, x.XQ.sB, x.XQ.sH, x.XQ.sL};
    a.k = TDesc{x.XK.data, x.XK.sB, x.XK.sH, x.XK.sL};
    a.v = TDesc{x.XV.data, x.XV.sB, x.XV.sH, x.XV.sL};
    a.eta = x.eta.data;
    a.eta_sB = x.eta.sB;
    a.eta_sH = x.eta.sH;
    a.te = x.eta.token_eta;
    a.ln_w = x.ln_w;
    a.ln_b = x.ln_b;
    a.W = st->W;
    a.b = st->b;
    a.Wg = st->W_grad;
    a.bg = st->b_grad;
    a.out = ODesc{x.out.data, x.out.sB, x.out.sH, x.out.sL};
    a.B = cfg->B;
    a.H = cfg->H;
    a.K = cfg->K;
    a.rope = cfg->rope;
    a.rope_base = cfg->rope_base;
    a.eps = cfg->ln_eps;
    a.grad_rows = cfg->grad_layout == TTT_GRAD_ROWS;
    return a;
}

ttt_status hip_fail(hipError_t e, const char *what) {
    return fail(TTT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A launch's error is read with hipGetLastError, which would also return an
// error left by an earlier, unrelated HIP call on this thread.  Such an error
// is taken (and cleared) before the first launch of a call, so the call
// reports it with nothing enqueued.
ttt_status take_pending_error() {
    if (hipError_t e = hipGetLastError(); e != hipSuccess)
        return fail(TTT_ERR_HIP, "an earlier HIP call on this thread left an error (%s); nothing was enqueued",
                    hipGetErrorString(e));
    return TTT_OK;
}

// A call made of several launches that fails after some of them were
// enqueued: the state has advanced by the tokens of those pieces.
ttt_status piece_fail(hipError_t e, const char *what, int64_t *offset, int done) {
    *offset += done;
    return fail(TTT_ERR_HIP, "%s: %s (the state advanced by the %d tokens already enqueued)", what,
                hipGetErrorString(e), done);
}

enum class Mode { Prefill, Decode };

ttt_status linear_call(Mode mode, const ttt_linear_cfg *cfg, int32_t L, const Act &x, ttt_linear_state *st,
                       void *stream) {
    if (!cfg) return fail(TTT_ERR_NULL, "cfg is NULL");
    ttt_status s;
    if ((s = check_common(cfg->B, cfg->H, cfg->D, cfg->K, cfg->in_dtype, cfg->out_dtype, cfg->ln_eps,
                          cfg->rope_base, cfg->rope)))
        return s;
    if (L < 1) return fail(TTT_ERR_SHAPE, "token count %d must be >= 1", L);
    if (cfg->grad_layout != TTT_GRAD_DENSE && cfg->grad_layout != TTT_GRAD_ROWS)
        return fail(TTT_ERR_UNSUPPORTED, "unknown grad_layout %d", (int)cfg->grad_layout);
    std::vector<Range> sr;
    if ((s = check_linear_state(cfg, st, sr))) return s;
    if ((s = check_acts(x, cfg->B, cfg->H, L, cfg->D, cfg->K, cfg->in_dtype, cfg->out_dtype, sr))) return s;

    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const int in_bf16 = cfg->in_dtype == TTT_BF16, out_bf16 = cfg->out_dtype == TTT_BF16;
    const int K = cfg->K;
    int head = 0, body = 0, tail = L;
    if (mode == Mode::Prefill && K == 16) {
        head = (int)std::min<int64_t>(L, (K - st->offset % K) % K);
        body = (L - head) / K;
        tail = L - head - body * K;
    }
    LinearArgs a = linear_args(cfg, x, st);
    if ((s = take_pending_error())) return s;
    hipError_t e;
    if (head > 0) {
        a.ntok = head;
        a.t0 = 0;
        a.pos0 = st->offset;
        if ((e = launch_linear_token(a, in_bf16, out_bf16, hs)) != hipSuccess) return hip_fail(e, "token kernel");
    }
    if (body > 0) {
        a.ntok = body;
        a.t0 = head;
        a.pos0 = st->offset + head;
        // the dual kernel addresses the rows of one mini-batch with 32-bit
        // byte offsets from a per-mini-batch base
        const int64_t rows = K;
        const size_t ei = dtype_size(cfg->in_dtype), eo = dtype_size(cfg->out_dtype);
        const int64_t span = std::max({(rows - 1) * x.XQ.sL * (int64_t)ei, (rows - 1) * x.XK.sL * (int64_t)ei,
                                       (rows - 1) * x.XV.sL * (int64_t)ei, (rows - 1) * x.out.sL * (int64_t)eo}) +
                             (int64_t)cfg->D * 4;
        if (span < (int64_t)INT32_MAX) {
            if ((e = launch_linear_dual(a, in_bf16, out_bf16, hs)) != hipSuccess)
                return piece_fail(e, "dual kernel", &st->offset, head);
        } else {
            a.ntok = body * K;  // token by token: same result, no 32-bit offsets
            if ((e = launch_linear_token(a, in_bf16, out_bf16, hs)) != hipSuccess)
                return piece_fail(e, "token kernel", &st->offset, head);
        }
    }
    if (tail > 0) {
        a.ntok = tail;
        a.t0 = L - tail;
        a.pos0 = st->offset + (L - tail);
        if ((e = launch_linear_token(a, in_bf16, out_bf16, hs)) != hipSuccess)
            return piece_fail(e, "token kernel", &st->offset, L - tail);
    }
    st->offset += L;
    return ok();
}

// TTT-MLP call: tokens that complete an open mini-batch run in the token
// kernel, whole mini-batches (and a trailing partial one) in the dual-form
// kernel; decode calls, fp32 inputs and K != 16 run token by token.
ttt_status mlp_call(Mode mode, const ttt_mlp_cfg *cfg, int32_t L, const Act &x, ttt_mlp_state *st,
                    void *stream) {
    ttt_status s;
    if ((s = check_mlp_cfg(cfg))) return s;
    if (L < 1) return fail(TTT_ERR_SHAPE, "token count %d must be >= 1", L);
    std::vector<Range> sr;
    if ((s = check_mlp_state(cfg, st, sr, true))) return s;
    if ((s = check_acts(x, cfg->B, cfg->H, L, cfg->D, cfg->K, cfg->in_dtype, cfg->out_dtype, sr))) return s;
    MlpArgs a{};
    a.q = TDesc{x.XQ.data, x.XQ.sB, x.XQ.sH, x.XQ.sL};
    a.k = TDesc{x.XK.data, x.XK.sB, x.XK.sH, x.XK.sL};
    a.v = TDesc{x.XV.data, x.XV.sB, x.XV.sH, x.XV.sL};
    a.eta = x.eta.data;
    a.eta_sB = x.eta.sB;
    a.eta_sH = x.eta.sH;
    a.te = x.eta.token_eta;
    a.ln_w = x.ln_w;
    a.ln_b = x.ln_b;
    a.W1 = st->W1;
    a.b1 = st->b1;
    a.W2 = st->W2;
    a.b2 = st->b2;
    a.W1g = st->W1_grad;
    a.b1g = st->b1_grad;
    a.W2g = st->W2_grad;
    a.b2g = st->b2_grad;
    a.out = ODesc{x.out.data, x.out.sB, x.out.sH, x.out.sL};
    a.B = cfg->B;
    a.H = cfg->H;
    a.K = cfg->K;
    a.rope = cfg->rope;
    a.rope_base = cfg->rope_base;
    a.eps = cfg->ln_eps;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const int in_bf16 = cfg->in_dtype == TTT_BF16, out_bf16 = cfg->out_dtype == TTT_BF16;
    a.grad_rows = cfg->grad_layout == TTT_GRAD_ROWS;
    const int K = cfg->K;
    // token kernel for `head` tokens, the dual kernel for `body` tokens, the
    // token kernel again for `tail` (the dual kernel leaves a trailing open
    // mini-batch in the dense layout only)
    int head = L, body = 0, tail = 0;
    if (mode == Mode::Prefill && K == 16 && in_bf16) {
        head = (int)std::min<int64_t>(L, (K - st->offset % K) % K);
        body = L - head;
        if (a.grad_rows) {
            tail = body % K;
            body -= tail;
        }
    }
    if ((s = take_pending_error())) return s;
    hipError_t e;
    if (head > 0) {
        a.ntok = head;
        a.t0 = 0;
        a.pos0 = st->offset;
        if ((e = launch_mlp_token(a, in_bf16, out_bf16, hs)) != hipSuccess) return hip_fail(e, "mlp token kernel");
    }
    if (body > 0) {
        a.nblk = (body + K - 1) / K;
        a.tail = body % K;
        a.t0 = head;
        a.pos0 = st->offset + head;
        if ((e = launch_mlp_dual(a, in_bf16, out_bf16, hs)) != hipSuccess)
            return piece_fail(e, "mlp kernel", &st->offset, head);
    }
    if (tail > 0) {
        a.ntok = tail;
        a.t0 = L - tail;
        a.pos0 = st->offset + (L - tail);
        if ((e = launch_mlp_token(a, in_bf16, out_bf16, hs)) != hipSuccess)
            return piece_fail(e, "mlp token kernel", &st->offset, L - tail);
    }
    st->offset += L;
    return ok();
}

}  // namespace

extern "C" {

const char *ttt_status_string(ttt_status s) {
    switch (s) {
    case TTT_OK: return "TTT_OK";
    case TTT_ERR_NULL: return "TTT_ERR_NULL";
    case TTT_ERR_SHAPE: return "TTT_ERR_SHAPE";
    case TTT_ERR_DTYPE: return "TTT_ERR_DTYPE";
    case TTT_ERR_ALIGN: return "TTT_ERR_ALIGN";
    case TTT_ERR_ALIAS: return "TTT_ERR_ALIAS";
    case TTT_ERR_STATE: return "TTT_ERR_STATE";
    case TTT_ERR_UNSUPPORTED: return "TTT_ERR_UNSUPPORTED";
    case TTT_ERR_HIP: return "TTT_ERR_HIP";
    }
    return "TTT_ERR_UNKNOWN";
}

const char *ttt_last_error(void) { return g_last_error.c_str(); }

ttt_status ttt_linear_state_init(const ttt_linear_cfg *cfg, const float *W0, const float *b0,
                                 ttt_linear_state *state, void *stream) {
    if (!cfg) return fail(TTT_ERR_NULL, "cfg is NULL");
    ttt_status s;
    if ((s = check_common(cfg->B, cfg->H, cfg->D, cfg->K, cfg->in_dtype, cfg->out_dtype, cfg->ln_eps,
                          cfg->rope_base, cfg->rope)))
        return s;
    if (!W0 || !b0) return fail(TTT_ERR_NULL, "W0 / b0 is NULL");
    std::vector<Range> sr;
    if ((s = check_linear_state(cfg, state, sr, false))) return s;
    const int64_t H = cfg->H, D = cfg->D, n = (int64_t)cfg->B * H;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    TileList t{};
    t.seg[0] = TileSeg{state->W, W0, H * D * D, n * D * D};
    t.seg[1] = TileSeg{state->b, b0, H * D, n * D};
    t.seg[2] = TileSeg{state->W_grad, nullptr, 1, n * D * D};
    t.seg[3] = TileSeg{state->b_grad, nullptr, 1, n * D};
    t.n = 4;
    if ((s = take_pending_error())) return s;
    if (hipError_t e = launch_tiles(t, hs); e != hipSuccess) return hip_fail(e, "state init");
    state->offset = 0;
    return ok();
}

ttt_status ttt_linear_prefill(const ttt_linear_cfg *cfg, int32_t L, ttt_tensor XQ, ttt_tensor XK, ttt_tensor XV,
                              ttt_eta eta, const float *ln_w, const float *ln_b, ttt_linear_state *state,
                              ttt_tensor out, void *stream) {
    return linear_call(Mode::Prefill, cfg, L, Act{XQ, XK, XV, out, eta, ln_w, ln_b}, state, stream);
}

ttt_status ttt_linear_decode(const ttt_linear_cfg *cfg, int32_t T, ttt_tensor XQ, ttt_tensor XK, ttt_tensor XV,
                             ttt_eta eta, const float *ln_w, const float *ln_b, ttt_linear_state *state,
                             ttt_tensor out, void *stream) {
    return linear_call(Mode::Decode, cfg, T, Act{XQ, XK, XV, out, eta, ln_w, ln_b}, state, stream);
}

ttt_status ttt_mlp_state_init(const ttt_mlp_cfg *cfg, const float *W1, const float *b1, const float *W2,
                              const float *b2, ttt_mlp_state *state, void *stream) {
    ttt_status s;
    if ((s = check_mlp_cfg(cfg))) return s;
    if (!W1 || !b1 || !W2 || !b2) return fail(TTT_ERR_NULL, "W1 / b1 / W2 / b2 is NULL");
    std::vector<Range> sr;
    if ((s = check_mlp_state(cfg, state, sr, false))) return s;
    const int64_t H = cfg->H, D = cfg->D, F = cfg->F, n = (int64_t)cfg->B * H;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    TileList t{};
    t.seg[0] = TileSeg{state->W1, W1, H * D * F, n * D * F};
    t.seg[1] = TileSeg{state->b1, b1, H * F, n * F};
    t.seg[2] = TileSeg{state->W2, W2, H * F * D, n * F * D};
    t.seg[3] = TileSeg{state->b2, b2, H * D, n * D};
    t.seg[4] = TileSeg{state->W1_grad, nullptr, 1, n * D * F};
    t.seg[5] = TileSeg{state->b1_grad, nullptr, 1, n * F};
    t.seg[6] = TileSeg{state->W2_grad, nullptr, 1, n * F * D};
    t.seg[7] = TileSeg{state->b2_grad, nullptr, 1, n * D};
    t.n = 8;
    if ((s = take_pending_error())) return s;
    if (hipError_t e = launch_tiles(t, hs); e != hipSuccess) return hip_fail(e, "state init");
    state->offset = 0;
    return ok();
}

ttt_status ttt_mlp_prefill(const ttt_mlp_cfg *cfg, int32_t L, ttt_tensor XQ, ttt_tensor XK, ttt_tensor XV,
                           ttt_eta eta, const float *ln_w, const float *ln_b, ttt_mlp_state *state, ttt_tensor out,
                           void *stream) {
    return mlp_call(Mode::Prefill, cfg, L, Act{XQ, XK, XV, out, eta, ln_w, ln_b}, state, stream);
}

ttt_status ttt_mlp_decode(const ttt_mlp_cfg *cfg, int32_t T, ttt_tensor XQ, ttt_tensor XK, ttt_tensor XV,
                          ttt_eta eta, const float *ln_w, const float *ln_b, ttt_mlp_state *state, ttt_tensor out,
                          void *stream) {
    return mlp_call(Mode::Decode, cfg, T, Act{XQ, XK, XV, out, eta, ln_w, ln_b}, state, stream);
}

size_t ttt_post_proj_prepared_bytes(int32_t K, int32_t N) {
    if (K <= 0 || N <= 0) return 0;
    return (size_t)K * (size_t)N * 2 + (size_t)N * 8;
}

ttt_status ttt_post_proj_prepare(int32_t K, int32_t N, const float *gamma, const float *beta, const float *Wo,
                                 const float *bias, void *prepared, void *stream) {
    if (!gamma || !beta || !Wo || !prepared) return fail(TTT_ERR_NULL, "gamma / beta / Wo / prepared is NULL");
    if (K < 64 || K % 64 || N < 256 || N % 256)
        return fail(TTT_ERR_SHAPE, "K = %d must be a positive multiple of 64 and N = %d of 256", K, N);
    if (!aligned16(prepared)) return fail(TTT_ERR_ALIGN, "prepared is not 16-byte aligned");
    const Range rp = flat_range(prepared, (int64_t)ttt_post_proj_prepared_bytes(K, N), 1);
    const Range ins[] = {flat_range(gamma, K, 4), flat_range(beta, K, 4), flat_range(Wo, (int64_t)K * N, 4),
                         bias ? flat_range(bias, N, 4) : Range{0, 0}};
    for (const Range &r : ins)
        if (overlap(rp, r)) return fail(TTT_ERR_ALIAS, "prepared overlaps an input");
    ttt_status s;
    if ((s = take_pending_error())) return s;
    PostPrepArgs a{};
    a.gamma = gamma;
    a.beta = beta;
    a.Wo = Wo;
    a.bias = bias;
    a.Wt = static_cast<__bf16 *>(prepared);
    a.c1 = reinterpret_cast<float *>(static_cast<char *>(prepared) + (size_t)K * N * 2);
    a.c2 = a.c1 + N;
    a.K = K;
    a.N = N;
    if (hipError_t e = launch_post_proj_prepare(a, reinterpret_cast<hipStream_t>(stream)); e != hipSuccess)
        return hip_fail(e, "post_proj prepare");
    return ok();
}

ttt_status ttt_post_proj(int32_t M, int32_t K, int32_t N, const void *y, int64_t ldy, float eps,
                         const void *prepared, void *out, int64_t ldo, int32_t out_dtype, void *stream) {
    if (!y || !prepared || !out) return fail(TTT_ERR_NULL, "y / prepared / out is NULL");
    if (M < 1 || K < 64 || K % 64 || N < 256 || N % 256)
        return fail(TTT_ERR_SHAPE, "M = %d must be >= 1, K = %d a positive multiple of 64, N = %d of 256", M, K, N);
    if (ldy < K || ldo < N) return fail(TTT_ERR_SHAPE, "row strides ldy = %lld < K or ldo = %lld < N",
                                        (long long)ldy, (long long)ldo);
    if (!dtype_valid(out_dtype)) return fail(TTT_ERR_DTYPE, "out_dtype %d is not TTT_F32 or TTT_BF16", out_dtype);
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(TTT_ERR_SHAPE, "eps must be finite and > 0");
    const size_t eo = dtype_size(out_dtype);
    if (!aligned16(y) || ldy % 8) return fail(TTT_ERR_ALIGN, "y must be 16-byte aligned with ldy a multiple of 8");
    if (!aligned16(prepared)) return fail(TTT_ERR_ALIGN, "prepared is not 16-byte aligned");
    if (!aligned16(out) || (ldo * (int64_t)eo) % 16)
        return fail(TTT_ERR_ALIGN, "out must be 16-byte aligned with rows a multiple of 16 bytes apart");
    const Range ry = flat_range(y, (int64_t)(M - 1) * ldy + K, 2);
    const Range rp = flat_range(prepared, (int64_t)ttt_post_proj_prepared_bytes(K, N), 1);
    const Range ro = flat_range(out, (int64_t)(M - 1) * ldo + N, eo);
    if (overlap(ro, ry) || overlap(ro, rp)) return fail(TTT_ERR_ALIAS, "out overlaps y or the prepared weights");
    ttt_status s;
    if ((s = take_pending_error())) return s;
    PostArgs a{};
    a.y = static_cast<const __bf16 *>(y);
    a.ldy = ldy;
    a.Wt = static_cast<const __bf16 *>(prepared);
    a.c1 = reinterpret_cast<const float *>(static_cast<const char *>(prepared) + (size_t)K * N * 2);
    a.c2 = a.c1 + N;
    a.out = out;
    a.ldo = ldo;
    a.M = M;
    a.K = K;
    a.N = N;
    a.eps = eps;
    if (hipError_t e = launch_post_proj(a, out_dtype == TTT_BF16, reinterpret_cast<hipStream_t>(stream));
        e != hipSuccess)
        return hip_fail(e, "post_proj");
    return ok();
}

}  // extern "C"
