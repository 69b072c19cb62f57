// api.hip -- the C ABI declared in include/linrec.h: argument checks, launch plans and
// kernel dispatch.  Host code only; every check runs before any HIP call.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <atomic>
#include <initializer_list>
#include <mutex>
#include <random>
#include <string>

#include "linrec.h"
#include "chunk_scan.hpp"
#include "wkv_backward.hpp"
#include "wkv_decode.hpp"
#include "token_shift.hpp"

#define LINREC_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return LINREC_OK;
}

// Optional integer override from the environment (tests use it to force launch shapes).
int64_t env_int(const char* name, int64_t dflt) {
    const char* s = std::getenv(name);
    if (!s || !*s) return dflt;
    char* end = nullptr;
    long long v = std::strtoll(s, &end, 10);
    return (end && *end == 0 && v > 0) ? (int64_t)v : dflt;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// B, T, C >= 0 and B*T*C*elem_bytes representable.
int check_shape(int64_t B, int64_t T, int64_t C, int64_t elem_bytes) {
    if (B < 0 || T < 0 || C < 0)
        return fail(LINREC_ERR_INVALID_ARG, "negative size: B=%lld T=%lld C=%lld", (long long)B,
                    (long long)T, (long long)C);
    int64_t n = 0;
    if (__builtin_mul_overflow(B, T, &n) || __builtin_mul_overflow(n, C, &n) ||
        __builtin_mul_overflow(n, elem_bytes, &n))
        return fail(LINREC_ERR_INVALID_ARG, "B*T*C*%lld bytes overflows int64", (long long)elem_bytes);
    return LINREC_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Launch plan of the forward scans for a given vector width; a pure function of
// (kind, vec, B, T, C) and the environment overrides (tests use them to force shapes).
linrec::ScanPlan scan_plan(int kind, int vec, int64_t B, int64_t T, int64_t C) {
    linrec::ScanPlan p{};
    p.vec = vec;
    // Default shapes, measured on MI355X at the workloads of the tests and the bench: WKV
    // is arithmetic-heavy and favours occupancy (fewer registers per lane), the scans
    // favour wider rows; long single sequences favour longer slabs (shorter look-backs).
    if (kind == linrec::kKindWkv) {
        p.nw = 8;
        p.L = 16;
    } else if (kind == linrec::kKindReal || kind == linrec::kKindMinGru || kind == linrec::kKindMinLstm ||
               kind == linrec::kKindRealDecay) {
        p.nw = 8;
        p.L = 16;
    } else if (kind == linrec::kKindRealBwd || kind == linrec::kKindMinGruBwd || kind == linrec::kKindMinLstmBwd ||
               kind == linrec::kKindRealDecayBwd || kind == linrec::kKindComplexNormBwd) {
        // The normalised LRU's adjoint also holds u per step: 32-step chunks would spill.
        p.nw = 8;
        p.L = 16;
    } else {
        // Complex (and its adjoint): one channel per lane over 32-step chunks (slabs of 256
        // steps) halves the look-back chains of a single long sequence; two channels per lane
        // take 16 steps.
        p.nw = 8;
        p.L = vec == 1 ? 32 : 16;
    }
    // Coordination: in wave 0 by default; in a wave of its own for the complex scans, whose
    // chunks hold many registers and whose long chains lean on the inclusive prefixes
    // (LINREC_COORD: 1 wave 0, 2 own wave).
    p.sep = vec == 1 && (kind == linrec::kKindComplex || kind == linrec::kKindComplexBwd ||
                         kind == linrec::kKindComplexNorm || kind == linrec::kKindComplexNormBwd);
    const int64_t coord = env_int("LINREC_COORD", 0);
    if (coord == 1 || coord == 2) p.sep = vec == 1 && coord == 2;
    const int nw = (int)env_int("LINREC_NW", 0), L = (int)env_int("LINREC_L", 0);
    if (nw > 0 && L > 0 && linrec::scan_shape_supported(kind, vec, nw, L)) {
        p.nw = nw;
        p.L = L;
    }
    const int64_t cw = 64 * (int64_t)vec;
    const int64_t nwg = B * ceil_div(C, cw) * (p.nslab = ceil_div(T, (int64_t)p.nw * p.L));
    p.ws_bytes = 0;
    if (p.nslab > 1)
        p.ws_bytes = align256((size_t)nwg * 8) + 2 * align256((size_t)(nwg * cw) * linrec::agg_bytes(kind));
    if (linrec::has_parts(kind)) {  // per-slab glam sums and their first-stage sums
        const int64_t nk = ceil_div(p.nslab, linrec::kPartBlock);
        p.ws_bytes += align256((size_t)(nwg * cw) * 16) + align256((size_t)(B * nk * C) * 16);
    }
    return p;
}

int vmax_of(int kind) {
    if (linrec::is_bwd_kind(kind)) return 1;
    return (kind == linrec::kKindWkv || kind == linrec::kKindReal) ? 4 : 2;
}

// Channels per lane: the widest the alignment allows, narrowed by the default policy or by
// LINREC_VEC (tests and tuning).  Measured on MI355X: the real scan takes 2; the plain WKV
// forward takes 2 on calls of at least 2^25 elements, which run many rounds of workgroups
// and gain from 512-byte rows, and 1 on smaller ones, which must fit the chip in one round;
// the WKV forward with state or gate and the complex scan take 1.
int pick_vec(int kind, int vec_aligned, int64_t elems = 0, bool plain = false) {
    int vec = vec_aligned;
    const int64_t f = env_int("LINREC_VEC", 0);
    if (f == 1 || f == 2 || f == 4) {
        vec = f < vec ? (int)f : vec;
    } else if (kind == linrec::kKindWkv) {
        vec = (plain && elems >= ((int64_t)1 << 25) && vec >= 2) ? 2 : 1;
    } else if (kind == linrec::kKindComplex || kind == linrec::kKindComplexNorm) {
        vec = 1;
    } else {
        vec = vec < 2 ? vec : 2;  // the real scan and its gated variants
    }
    return vec;
}

// Workspace the caller must provide: enough for either vector width (the width depends on
// pointer alignment, which a size query does not see).
size_t scan_ws_bytes(int kind, int64_t B, int64_t T, int64_t C) {
    size_t best = 0;
    for (int vec : {vmax_of(kind), 2, 1}) {
        if (vec > vmax_of(kind)) continue;
        const size_t x = scan_plan(kind, vec, B, T, C).ws_bytes;
        best = x > best ? x : best;
    }
    return best;
}

// Per-call tag of the look-back flags: unique within the process and never 0.
uint64_t next_tag() {
    static std::atomic<uint64_t> counter{0};
    static const uint64_t salt = [] {
        std::random_device rd;
        return ((uint64_t)rd() << 32) ^ (uint64_t)rd();
    }();
    uint64_t t = (salt + counter.fetch_add(1, std::memory_order_relaxed)) & ((1ull << 61) - 1);
    return t ? t : 1;
}

// Backward plan for a vector width; LINREC_BWD_NW / LINREC_BWD_L override the slab shape.
linrec::BwdPlan bwd_plan(int vec, int64_t B, int64_t T, int64_t C) {
    return linrec::wkv_backward_plan(vec, B, T, C, (int)env_int("LINREC_BWD_NW", 0), (int)env_int("LINREC_BWD_L", 0));
}

size_t bwd_ws_bytes(int64_t B, int64_t T, int64_t C) { return bwd_plan(1, B, T, C).ws_bytes; }

int spin_limit() {
    // Polls (each ~128 cycles) before a missing predecessor aggregate is recomputed;
    // LINREC_SPIN overrides it (0 forces the recompute path, for tests).
    const char* spin = std::getenv("LINREC_SPIN");
    return (spin && *spin) ? (int)std::strtol(spin, nullptr, 10) : 4096;
}

linrec::ScanGeom geom_of(int kind, const linrec::ScanPlan& p, int64_t B, int64_t T, int64_t C, void* ws) {
    linrec::ScanGeom g{};
    g.B = B;
    g.T = T;
    g.C = C;
    const int64_t cw = 64 * (int64_t)p.vec;
    g.ngrp = ceil_div(C, cw);
    g.nslab = p.nslab;
    g.tag = next_tag();
    g.spin = spin_limit();
    const int64_t nwg = B * g.ngrp * g.nslab;
    g.flags = reinterpret_cast<uint64_t*>(ws);
    char* rec = (char*)ws + align256((size_t)nwg * 8);
    g.rec_agg = rec;
    g.rec_incl = rec + align256((size_t)(nwg * cw) * linrec::agg_bytes(kind));
    char* after = (char*)g.rec_incl + align256((size_t)(nwg * cw) * linrec::agg_bytes(kind));
    if (p.nslab <= 1) g.flags = nullptr, g.rec_agg = g.rec_incl = nullptr, after = (char*)ws;
    g.part = g.part2 = nullptr;
    g.nk = ceil_div(g.nslab, linrec::kPartBlock);
    if (linrec::has_parts(kind)) {
        g.part = reinterpret_cast<double*>(after);
        g.part2 = reinterpret_cast<double*>(after + align256((size_t)(nwg * cw) * 16));
    }
    return g;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (ws_bytes < need)
        return fail(LINREC_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
    if (need > 0 && ws == nullptr) return fail(LINREC_ERR_INVALID_ARG, "workspace is NULL");
    if (need > 0 && !aligned(ws, 16)) return fail(LINREC_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
    return LINREC_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

LINREC_API int linrec_abi_version(void) { return LINREC_ABI_VERSION; }

LINREC_API const char* linrec_status_string(int status) {
    switch (status) {
        case LINREC_OK: return "LINREC_OK";
        case LINREC_ERR_INVALID_ARG: return "LINREC_ERR_INVALID_ARG";
        case LINREC_ERR_WORKSPACE: return "LINREC_ERR_WORKSPACE";
        case LINREC_ERR_UNSUPPORTED: return "LINREC_ERR_UNSUPPORTED";
        case LINREC_ERR_HIP: return "LINREC_ERR_HIP";
        default: return "unknown status";
    }
}

LINREC_API const char* linrec_last_error(void) { return g_last_error.c_str(); }

LINREC_API size_t wkv4_forward_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || B == 0 || T == 0 || C == 0) return 0;
    return scan_ws_bytes(linrec::kKindWkv, B, T, C);
}

LINREC_API size_t linrec_scan_workspace_size(int64_t B, int64_t T, int64_t C, int is_complex) {
    if (B < 0 || T < 0 || C < 0 || B == 0 || T == 0 || C == 0) return 0;
    return scan_ws_bytes(is_complex ? linrec::kKindComplex : linrec::kKindReal, B, T, C);
}

LINREC_API size_t linrec_scan_backward_workspace_size(int64_t B, int64_t T, int64_t C, int is_complex) {
    if (B < 0 || T < 0 || C < 0 || B == 0 || T == 0 || C == 0) return 0;
    // Enough for every adjoint of the family (the plain scan's and its variants').
    size_t best = 0;
    const int real_kinds[] = {linrec::kKindRealBwd, linrec::kKindMinGruBwd, linrec::kKindMinLstmBwd,
                              linrec::kKindRealDecayBwd};
    const int cplx_kinds[] = {linrec::kKindComplexBwd, linrec::kKindComplexNormBwd};
    if (is_complex) {
        for (int k : cplx_kinds) best = std::max(best, scan_ws_bytes(k, B, T, C));
    } else {
        for (int k : real_kinds) best = std::max(best, scan_ws_bytes(k, B, T, C));
    }
    return best;
}

LINREC_API size_t wkv4_backward_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || B == 0 || T == 0 || C == 0) return 0;
    return bwd_ws_bytes(B, T, C);
}

LINREC_API int wkv4_forward_ex(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                               const float* k, const float* v, const float* r, const float* s_in, float* y,
                               float* s_out, void* workspace, size_t ws_bytes, void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (B == 0 || C == 0) return ok();
    if ((s_in && !aligned(s_in, 4)) || (s_out && !aligned(s_out, 4)))
        return fail(LINREC_ERR_UNSUPPORTED, "state pointer not 4-byte aligned");
    if (T == 0) {
        // No tokens: the state passes through unchanged (empty without s_in).
        if (!s_out) return ok();
        const hipError_t e = s_in ? linrec::run_copy(s_out, s_in, 3 * B * C, (hipStream_t)stream)
                                  : linrec::run_fill_zero(s_out, 3 * B * C, (hipStream_t)stream);
        return hip_status(e, "wkv4_forward_ex state copy");
    }
    if (!w || !u || !k || !v || !y) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {w, u, k, v, y};
    for (const void* p : ptrs)
        if (!aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    if (r && !aligned(r, 4)) return fail(LINREC_ERR_UNSUPPORTED, "r not 4-byte aligned");
    const bool wide_ok = !r || aligned(r, 16);
    const int vec = pick_vec(linrec::kKindWkv,
                             (C % 4 == 0 && aligned(k, 16) && aligned(v, 16) && aligned(y, 16) && wide_ok) ? 4
                             : (C % 2 == 0 && aligned(k, 8) && aligned(v, 8) && aligned(y, 8) && (!r || aligned(r, 8))) ? 2
                                                                                                            : 1,
                             B * T * C, !r && !s_in && !s_out);
    const linrec::ScanPlan p = scan_plan(linrec::kKindWkv, vec, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    const linrec::WkvArgs A{w, u, k, v, y, env_int("LINREC_WKV_EXACT", 0) > 0 ? 1 : 0, r, s_in, s_out};
    return hip_status(linrec::run_wkv_forward(A, geom_of(linrec::kKindWkv, p, B, T, C, workspace), p,
                                              (hipStream_t)stream),
                      "wkv4_forward launch");
}

LINREC_API int wkv4_forward(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                            const float* k, const float* v, float* y, void* workspace,
                            size_t ws_bytes, void* stream) {
    return wkv4_forward_ex(B, T, C, w, u, k, v, nullptr, nullptr, y, nullptr, workspace, ws_bytes, stream);
}

LINREC_API int rwkv_token_shift(int64_t B, int64_t T, int64_t C, int64_t M, const float* x, const float* x_prev,
                                const float* mu, float* out, void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (M < 1 || M > linrec::kShiftMaxM) return fail(LINREC_ERR_INVALID_ARG, "M must be 1..%d", linrec::kShiftMaxM);
    if ((st = check_shape(M, B * T, C, 4))) return st;
    if (B == 0 || T == 0 || C == 0) return ok();
    if (!x || !mu || !out) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {x, x_prev, mu, out};
    for (const void* p : ptrs)
        if (p && !aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    const bool a16 = aligned(x, 16) && aligned(out, 16) && (!x_prev || aligned(x_prev, 16));
    const bool a8 = aligned(x, 8) && aligned(out, 8) && (!x_prev || aligned(x_prev, 8));
    // Two channels per lane measured fastest (B8 T1024 C768, 3 mixes: 17.9 us vs 18.6 for
    // four, 20.1 for one); LINREC_VEC forces 1, 2 or 4 where the alignment allows.
    const int vmax = (C % 4 == 0 && a16) ? 4 : ((C % 2 == 0 && a8) ? 2 : 1);
    int vec = vmax < 2 ? vmax : 2;
    const int64_t f = env_int("LINREC_VEC", 0);
    if ((f == 1 || f == 2 || f == 4) && f <= vmax) vec = (int)f;
    const linrec::TokenShiftArgs A{x, x_prev, mu, out};
    return hip_status(linrec::run_token_shift(A, B, T, C, (int)M, vec, (hipStream_t)stream), "rwkv_token_shift launch");
}

LINREC_API size_t rwkv_token_shift_backward_workspace_size(int64_t B, int64_t T, int64_t C, int64_t M) {
    if (check_shape(B, T, C, 4) || M < 1 || M > linrec::kShiftMaxM || B == 0 || T == 0 || C == 0) return 0;
    // Enough for either lane width (the width depends on pointer alignment).
    const size_t a = linrec::token_shift_backward_ws_bytes(B, T, C, (int)M, 1);
    const size_t b = linrec::token_shift_backward_ws_bytes(B, T, C, (int)M, 2);
    return align256(a > b ? a : b);
}

LINREC_API int rwkv_token_shift_backward(int64_t B, int64_t T, int64_t C, int64_t M, const float* x,
                                         const float* x_prev, const float* mu, const float* g, float* gx,
                                         float* gmu, float* gx_prev, void* workspace, size_t ws_bytes,
                                         void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (M < 1 || M > linrec::kShiftMaxM) return fail(LINREC_ERR_INVALID_ARG, "M must be 1..%d", linrec::kShiftMaxM);
    if ((st = check_shape(M, B * T, C, 4))) return st;
    if (C == 0) return ok();
    if (B == 0 || T == 0) {
        // Sums over an empty batch or sequence: zero.
        if (!gmu) return fail(LINREC_ERR_INVALID_ARG, "gmu is NULL");
        if (!aligned(gmu, 4) || (gx_prev && !aligned(gx_prev, 4)))
            return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
        hipError_t e = linrec::run_fill_zero(gmu, M * C, (hipStream_t)stream);
        if (e == hipSuccess && gx_prev && B > 0) e = linrec::run_fill_zero(gx_prev, B * C, (hipStream_t)stream);
        return hip_status(e, "rwkv_token_shift_backward zero fill");
    }
    if (!x || !mu || !g || !gx || !gmu) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {x, x_prev, mu, g, gx, gmu, gx_prev};
    for (const void* p : ptrs)
        if (p && !aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    if ((st = check_ws(workspace, ws_bytes, rwkv_token_shift_backward_workspace_size(B, T, C, M)))) return st;
    const bool a8 = aligned(x, 8) && aligned(g, 8) && aligned(gx, 8) && (!x_prev || aligned(x_prev, 8));
    int vec = (C % 2 == 0 && a8) ? 2 : 1;
    if (env_int("LINREC_VEC", 0) == 1) vec = 1;
    const linrec::TokenShiftBwdArgs A{x, x_prev, mu, g, gx, gmu, gx_prev, reinterpret_cast<double*>(workspace)};
    return hip_status(linrec::run_token_shift_backward(A, B, T, C, (int)M, vec, (hipStream_t)stream),
                      "rwkv_token_shift_backward launch");
}

LINREC_API int wkv4_decode_step(int64_t B, int64_t C, const float* w, const float* u, const float* k,
                                const float* v, const float* r, float* state, float* y, void* stream) {
    int st = check_shape(B, 3, C, 4);
    if (st) return st;
    if (B == 0 || C == 0) return ok();
    if (!w || !u || !k || !v || !state || !y) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {w, u, k, v, r, state, y};
    for (const void* p : ptrs)
        if (p && !aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    const linrec::WkvStepArgs A{w, u, k, v, r, state, y};
    return hip_status(linrec::run_wkv_decode_step(A, B, C, (hipStream_t)stream), "wkv4_decode_step launch");
}

LINREC_API int linrec_scan_real(int64_t B, int64_t T, int64_t C, const float* a, const float* b,
                                const float* x0, float* x, void* workspace, size_t ws_bytes,
                                void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (B == 0 || T == 0 || C == 0) return ok();
    if (!a || !b || !x) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {a, b, x};
    for (const void* p : ptrs)
        if (!aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    if (x0 && !aligned(x0, 4)) return fail(LINREC_ERR_UNSUPPORTED, "x0 not 4-byte aligned");
    const int vec = pick_vec(linrec::kKindReal, (C % 4 == 0 && aligned(a, 16) && aligned(b, 16) && aligned(x, 16)) ? 4
                                               : (C % 2 == 0 && aligned(a, 8) && aligned(b, 8) && aligned(x, 8)) ? 2
                                                                                                            : 1);
    const linrec::ScanPlan p = scan_plan(linrec::kKindReal, vec, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    const linrec::RealArgs A{a, b, x0, x};
    return hip_status(linrec::run_scan_real(A, geom_of(linrec::kKindReal, p, B, T, C, workspace), p,
                                            (hipStream_t)stream),
                      "linrec_scan_real launch");
}

LINREC_API int linrec_scan_complex(int64_t B, int64_t T, int64_t C, const float* lambda,
                                   const float* u, const float* x0, float* x, void* workspace,
                                   size_t ws_bytes, void* stream) {
    int st = check_shape(B, T, C, 8);
    if (st) return st;
    if (B == 0 || T == 0 || C == 0) return ok();
    if (!lambda || !u || !x) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {lambda, u, x};
    for (const void* p : ptrs)
        if (!aligned(p, 8)) return fail(LINREC_ERR_UNSUPPORTED, "complex64 pointer not 8-byte aligned");
    if (x0 && !aligned(x0, 8)) return fail(LINREC_ERR_UNSUPPORTED, "x0 not 8-byte aligned");
    const int vec = pick_vec(linrec::kKindComplex, (C % 2 == 0 && aligned(u, 16) && aligned(x, 16)) ? 2 : 1);
    const linrec::ScanPlan p = scan_plan(linrec::kKindComplex, vec, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    const linrec::CplxArgs A{lambda, u, x0, x};
    return hip_status(linrec::run_scan_complex(A, geom_of(linrec::kKindComplex, p, B, T, C, workspace), p,
                                               (hipStream_t)stream),
                      "linrec_scan_complex launch");
}

namespace {

// Shared checks and launch of the gated real-scan variants: `tensors` are the (B,T,C)
// inputs, `chan` an optional (C) input; vec from the alignment of all of them and of x.
template <class Args, class Run>
int gated_real_scan(const char* name, int kind, int64_t B, int64_t T, int64_t C, std::initializer_list<const float*> tensors,
                    const float* chan, const float* x0, float* x, void* workspace, size_t ws_bytes, void* stream,
                    const Args& A, Run&& run) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (B == 0 || T == 0 || C == 0) return ok();
    bool a16 = aligned(x, 16), a8 = aligned(x, 8);
    if (!x) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    for (const float* p : tensors) {
        if (!p) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
        a16 = a16 && aligned(p, 16);
        a8 = a8 && aligned(p, 8);
    }
    const void* ptrs[] = {chan, x0, x};
    for (const void* p : ptrs)
        if (p && !aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    for (const float* p : tensors)
        if (!aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    const int vec = pick_vec(kind, (C % 4 == 0 && a16) ? 4 : ((C % 2 == 0 && a8) ? 2 : 1));
    const linrec::ScanPlan p = scan_plan(kind, vec, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    return hip_status(run(A, geom_of(kind, p, B, T, C, workspace), p, (hipStream_t)stream), name);
}

}  // namespace

LINREC_API int linrec_scan_mingru(int64_t B, int64_t T, int64_t C, const float* kz, const float* h,
                                  const float* x0, float* x, void* workspace, size_t ws_bytes, void* stream) {
    const linrec::MinGruArgs A{kz, h, x0, x};
    return gated_real_scan("linrec_scan_mingru launch", linrec::kKindMinGru, B, T, C, {kz, h}, nullptr, x0, x,
                           workspace, ws_bytes, stream, A, linrec::run_scan_mingru);
}

LINREC_API int linrec_scan_minlstm(int64_t B, int64_t T, int64_t C, const float* kf, const float* ki,
                                   const float* h, const float* x0, float* x, void* workspace, size_t ws_bytes,
                                   void* stream) {
    const linrec::MinLstmArgs A{kf, ki, h, x0, x};
    return gated_real_scan("linrec_scan_minlstm launch", linrec::kKindMinLstm, B, T, C, {kf, ki, h}, nullptr, x0, x,
                           workspace, ws_bytes, stream, A, linrec::run_scan_minlstm);
}

LINREC_API int linrec_scan_real_decay(int64_t B, int64_t T, int64_t C, const float* lambda, const float* u,
                                      const float* x0, float* x, void* workspace, size_t ws_bytes, void* stream) {
    if (B > 0 && T > 0 && C > 0 && !lambda) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const linrec::RealDecayArgs A{lambda, u, x0, x};
    return gated_real_scan("linrec_scan_real_decay launch", linrec::kKindRealDecay, B, T, C, {u}, lambda, x0, x,
                           workspace, ws_bytes, stream, A, linrec::run_scan_real_decay);
}

LINREC_API int linrec_scan_complex_normalized(int64_t B, int64_t T, int64_t C, const float* lambda,
                                              const float* u, const float* x0, float* x, void* workspace,
                                              size_t ws_bytes, void* stream) {
    int st = check_shape(B, T, C, 8);
    if (st) return st;
    if (B == 0 || T == 0 || C == 0) return ok();
    if (!lambda || !u || !x) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {lambda, u, x};
    for (const void* p : ptrs)
        if (!aligned(p, 8)) return fail(LINREC_ERR_UNSUPPORTED, "complex64 pointer not 8-byte aligned");
    if (x0 && !aligned(x0, 8)) return fail(LINREC_ERR_UNSUPPORTED, "x0 not 8-byte aligned");
    const int vec = pick_vec(linrec::kKindComplexNorm, (C % 2 == 0 && aligned(u, 16) && aligned(x, 16)) ? 2 : 1);
    const linrec::ScanPlan p = scan_plan(linrec::kKindComplexNorm, vec, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    const linrec::CplxArgs A{lambda, u, x0, x};
    return hip_status(linrec::run_scan_complex_normalized(A, geom_of(linrec::kKindComplexNorm, p, B, T, C, workspace),
                                                          p, (hipStream_t)stream),
                      "linrec_scan_complex_normalized launch");
}

LINREC_API int linrec_scan_real_backward(int64_t B, int64_t T, int64_t C, const float* a, const float* x0,
                                         const float* x, const float* gx, float* ga, float* gb, float* gx0,
                                         void* workspace, size_t ws_bytes, void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (B == 0 || C == 0) return ok();
    if (gx0 && !aligned(gx0, 4)) return fail(LINREC_ERR_UNSUPPORTED, "gx0 not 4-byte aligned");
    if (T == 0) {
        // No steps: the gradient of the initial state is zero.
        if (!gx0) return ok();
        return hip_status(linrec::run_fill_zero(gx0, B * C, (hipStream_t)stream), "linrec_scan_real_backward zero-fill");
    }
    if (!a || !x || !gx || !ga || !gb) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {a, x, gx, ga, gb};
    for (const void* p : ptrs)
        if (!aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    if (x0 && !aligned(x0, 4)) return fail(LINREC_ERR_UNSUPPORTED, "x0 not 4-byte aligned");
    const linrec::ScanPlan p = scan_plan(linrec::kKindRealBwd, 1, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    const linrec::RealBwdArgs A{a, x0, x, gx, ga, gb, gx0};
    return hip_status(linrec::run_scan_real_backward(A, geom_of(linrec::kKindRealBwd, p, B, T, C, workspace), p,
                                                     (hipStream_t)stream),
                      "linrec_scan_real_backward launch");
}

LINREC_API int linrec_scan_complex_backward(int64_t B, int64_t T, int64_t C, const float* lambda,
                                            const float* x0, const float* x, const float* gx, float* glambda,
                                            float* gu, float* gx0, void* workspace, size_t ws_bytes,
                                            void* stream) {
    int st = check_shape(B, T, C, 8);
    if (st) return st;
    if (C == 0) return ok();
    if (!glambda) return fail(LINREC_ERR_INVALID_ARG, "glambda is NULL");
    if (!aligned(glambda, 8) || (gx0 && !aligned(gx0, 8)))
        return fail(LINREC_ERR_UNSUPPORTED, "complex64 pointer not 8-byte aligned");
    if (B == 0 || T == 0) {
        // Empty sums: glambda = 0, and the gradient of the initial state is zero.
        hipError_t e = linrec::run_fill_zero(glambda, 2 * C, (hipStream_t)stream);
        if (e == hipSuccess && gx0 && B > 0) e = linrec::run_fill_zero(gx0, 2 * B * C, (hipStream_t)stream);
        return hip_status(e, "linrec_scan_complex_backward zero-fill");
    }
    if (!lambda || !x || !gx || !gu) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {lambda, x, gx, gu};
    for (const void* p : ptrs)
        if (!aligned(p, 8)) return fail(LINREC_ERR_UNSUPPORTED, "complex64 pointer not 8-byte aligned");
    if (x0 && !aligned(x0, 8)) return fail(LINREC_ERR_UNSUPPORTED, "x0 not 8-byte aligned");
    const linrec::ScanPlan p = scan_plan(linrec::kKindComplexBwd, 1, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    const linrec::CplxBwdArgs A{lambda, x0, x, gx, gu, gx0};
    return hip_status(linrec::run_scan_complex_backward(A, glambda, geom_of(linrec::kKindComplexBwd, p, B, T, C, workspace),
                                                        p, (hipStream_t)stream),
                      "linrec_scan_complex_backward launch");
}

namespace {

// Shared checks and launch of the real variants' adjoints: `ins` are the (B,T,C) inputs,
// `outs` the (B,T,C) outputs; gx0 (B,C) optional.  With T = 0 only gx0 (zero) and glam
// (zero, real decay) are written.
template <class Args, class Run>
int gated_real_backward(const char* name, int kind, int64_t B, int64_t T, int64_t C,
                        std::initializer_list<const float*> ins, std::initializer_list<float*> outs,
                        const float* x0, float* gx0, float* glam, void* workspace, size_t ws_bytes, void* stream,
                        const Args& A, Run run) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (C == 0) return ok();
    if (kind == linrec::kKindRealDecayBwd && !glam) return fail(LINREC_ERR_INVALID_ARG, "glambda is NULL");
    if ((gx0 && !aligned(gx0, 4)) || (glam && !aligned(glam, 4)))
        return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    if (B == 0 || T == 0) {
        // Empty sums: glambda = 0, and the gradient of the initial state is zero.
        hipError_t e = hipSuccess;
        if (glam) e = linrec::run_fill_zero(glam, C, (hipStream_t)stream);
        if (e == hipSuccess && gx0 && B > 0) e = linrec::run_fill_zero(gx0, B * C, (hipStream_t)stream);
        return hip_status(e, name);
    }
    for (const float* p : ins)
        if (!p) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    for (const float* p : outs)
        if (!p) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    for (const float* p : ins)
        if (!aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    for (const float* p : outs)
        if (!aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    if (x0 && !aligned(x0, 4)) return fail(LINREC_ERR_UNSUPPORTED, "x0 not 4-byte aligned");
    const linrec::ScanPlan p = scan_plan(kind, 1, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    return hip_status(run(A, geom_of(kind, p, B, T, C, workspace), p, (hipStream_t)stream), name);
}

}  // namespace

LINREC_API int linrec_scan_mingru_backward(int64_t B, int64_t T, int64_t C, const float* kz, const float* h,
                                           const float* x0, const float* x, const float* gx, float* gkz, float* gh,
                                           float* gx0, void* workspace, size_t ws_bytes, void* stream) {
    const linrec::MinGruBwdArgs A{kz, h, x0, x, gx, gkz, gh, gx0};
    return gated_real_backward("linrec_scan_mingru_backward launch", linrec::kKindMinGruBwd, B, T, C, {kz, h, x, gx},
                               {gkz, gh}, x0, gx0, nullptr, workspace, ws_bytes, stream, A,
                               linrec::run_scan_mingru_backward);
}

LINREC_API int linrec_scan_minlstm_backward(int64_t B, int64_t T, int64_t C, const float* kf, const float* ki,
                                            const float* h, const float* x0, const float* x, const float* gx,
                                            float* gkf, float* gki, float* gh, float* gx0, void* workspace,
                                            size_t ws_bytes, void* stream) {
    const linrec::MinLstmBwdArgs A{kf, ki, h, x0, x, gx, gkf, gki, gh, gx0};
    return gated_real_backward("linrec_scan_minlstm_backward launch", linrec::kKindMinLstmBwd, B, T, C,
                               {kf, ki, h, x, gx}, {gkf, gki, gh}, x0, gx0, nullptr, workspace, ws_bytes, stream, A,
                               linrec::run_scan_minlstm_backward);
}

LINREC_API int linrec_scan_real_decay_backward(int64_t B, int64_t T, int64_t C, const float* lambda, const float* x0,
                                               const float* x, const float* gx, float* glambda, float* gu, float* gx0,
                                               void* workspace, size_t ws_bytes, void* stream) {
    const linrec::RealDecayBwdArgs A{lambda, x0, x, gx, gu, gx0};
    auto run = [glambda](const linrec::RealDecayBwdArgs& a, const linrec::ScanGeom& g, const linrec::ScanPlan& p,
                         hipStream_t st) { return linrec::run_scan_real_decay_backward(a, glambda, g, p, st); };
    return gated_real_backward("linrec_scan_real_decay_backward launch", linrec::kKindRealDecayBwd, B, T, C,
                               {lambda, x, gx}, {gu}, x0, gx0, glambda, workspace, ws_bytes, stream, A, run);
}

LINREC_API int linrec_scan_complex_normalized_backward(int64_t B, int64_t T, int64_t C, const float* lambda,
                                                       const float* u, const float* x0, const float* x,
                                                       const float* gx, float* glambda, float* gu, float* gx0,
                                                       void* workspace, size_t ws_bytes, void* stream) {
    int st = check_shape(B, T, C, 8);
    if (st) return st;
    if (C == 0) return ok();
    if (!glambda) return fail(LINREC_ERR_INVALID_ARG, "glambda is NULL");
    if (!aligned(glambda, 8) || (gx0 && !aligned(gx0, 8)))
        return fail(LINREC_ERR_UNSUPPORTED, "complex64 pointer not 8-byte aligned");
    if (B == 0 || T == 0) {
        hipError_t e = linrec::run_fill_zero(glambda, 2 * C, (hipStream_t)stream);
        if (e == hipSuccess && gx0 && B > 0) e = linrec::run_fill_zero(gx0, 2 * B * C, (hipStream_t)stream);
        return hip_status(e, "linrec_scan_complex_normalized_backward zero-fill");
    }
    if (!lambda || !u || !x || !gx || !gu) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {lambda, u, x, gx, gu};
    for (const void* p : ptrs)
        if (!aligned(p, 8)) return fail(LINREC_ERR_UNSUPPORTED, "complex64 pointer not 8-byte aligned");
    if (x0 && !aligned(x0, 8)) return fail(LINREC_ERR_UNSUPPORTED, "x0 not 8-byte aligned");
    const linrec::ScanPlan p = scan_plan(linrec::kKindComplexNormBwd, 1, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    const linrec::CplxBwdArgs A{lambda, x0, x, gx, gu, gx0, u};
    return hip_status(linrec::run_scan_complex_normalized_backward(
                          A, glambda, geom_of(linrec::kKindComplexNormBwd, p, B, T, C, workspace), p,
                          (hipStream_t)stream),
                      "linrec_scan_complex_normalized_backward launch");
}

LINREC_API int wkv4_backward_ex(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                                const float* k, const float* v, const float* r, const float* s_in,
                                const float* s_out, const float* gy, const float* gs_out, float* gw, float* gu,
                                float* gk, float* gv, float* gr, float* gs_in, void* workspace, size_t ws_bytes,
                                void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (C > 0 && (!gw || !gu)) return fail(LINREC_ERR_INVALID_ARG, "gw or gu is NULL");
    if ((r == nullptr) != (gr == nullptr)) return fail(LINREC_ERR_INVALID_ARG, "r and gr must be given together");
    if (gs_out && !s_out) return fail(LINREC_ERR_INVALID_ARG, "gs_out needs s_out (its exponents)");
    const void* sptrs[] = {s_in, s_out, gs_out, gs_in};
    for (const void* p : sptrs)
        if (p && !aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "state pointer not 4-byte aligned");
    const linrec::WkvBwdArgs A{w, u, k, v, gy, gw, gu, gk, gv, r, gr, s_in, s_out, gs_out, gs_in};
    if (B == 0 || T == 0 || C == 0) {
        // Empty batch or sequence: the per-channel sums dL/dw, dL/du are zero, and without
        // tokens the state passes through (dL/ds_in from dL/ds_out alone).
        if (C == 0) return ok();
        if (!aligned(gw, 4) || !aligned(gu, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
        hipError_t e = linrec::run_zero_wu(gw, gu, C, (hipStream_t)stream);
        if (e == hipSuccess && gs_in) e = linrec::run_state_grad_passthrough(A, B, C, (hipStream_t)stream);
        return hip_status(e, "wkv4_backward zero-fill");
    }
    if (!w || !u || !k || !v || !gy || !gk || !gv)
        return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {w, u, k, v, r, gy, gw, gu, gk, gv, gr};
    for (const void* p : ptrs)
        if (p && !aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    const linrec::BwdPlan p = bwd_plan(1, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    linrec::BwdGeom g{};
    g.B = B;
    g.T = T;
    g.C = C;
    g.ngrp = ceil_div(C, 64 * (int64_t)p.vec);
    g.nslab = p.nslab;
    g.spin = spin_limit();
    g.tag_f = next_tag();
    g.tag_r = next_tag();
    g.exact_only = env_int("LINREC_WKV_EXACT", 0) > 0 ? 1 : 0;
    linrec::wkv_backward_layout(p, B, C, workspace, g);
    return hip_status(linrec::run_wkv_backward(A, g, p, (hipStream_t)stream), "wkv4_backward launch");
}

LINREC_API size_t wkv4_checkpoint_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || B == 0 || T == 0 || C == 0) return 0;
    return linrec::wkv_ckpt_bytes(B, T, C);
}

LINREC_API size_t wkv4_forward_ckpt_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || B == 0 || T == 0 || C == 0) return 0;
    return linrec::wkv_ckpt_forward_ws_bytes(B, T, C);
}

LINREC_API size_t wkv4_backward_ckpt_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || B == 0 || T == 0 || C == 0) return 0;
    return linrec::wkv_backward_ckpt_ws_bytes(B, T, C);
}

namespace {
int check_ckpt(const void* ckpt, size_t ckpt_bytes, size_t need) {
    if (ckpt_bytes < need)
        return fail(LINREC_ERR_WORKSPACE, "checkpoint buffer of %zu bytes, need %zu", ckpt_bytes, need);
    if (ckpt == nullptr) return fail(LINREC_ERR_INVALID_ARG, "checkpoint buffer is NULL");
    if (!aligned(ckpt, 16)) return fail(LINREC_ERR_UNSUPPORTED, "checkpoint buffer not 16-byte aligned");
    return LINREC_OK;
}
}  // namespace

LINREC_API int wkv4_forward_ckpt_ex(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                                    const float* k, const float* v, const float* r, const float* s_in, float* y,
                                    float* s_out, void* ckpt, size_t ckpt_bytes, void* workspace, size_t ws_bytes,
                                    void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (B == 0 || C == 0) return ok();
    if ((s_in && !aligned(s_in, 4)) || (s_out && !aligned(s_out, 4)))
        return fail(LINREC_ERR_UNSUPPORTED, "state pointer not 4-byte aligned");
    if (T == 0) {
        // No tokens: nothing to keep; the state passes through unchanged (empty without s_in).
        if (!s_out) return ok();
        const hipError_t e = s_in ? linrec::run_copy(s_out, s_in, 3 * B * C, (hipStream_t)stream)
                                  : linrec::run_fill_zero(s_out, 3 * B * C, (hipStream_t)stream);
        return hip_status(e, "wkv4_forward_ckpt_ex state copy");
    }
    if (!w || !u || !k || !v || !y) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {w, u, k, v, y, r};
    for (const void* p : ptrs)
        if (p && !aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    if ((st = check_ckpt(ckpt, ckpt_bytes, linrec::wkv_ckpt_bytes(B, T, C)))) return st;
    if ((st = check_ws(workspace, ws_bytes, linrec::wkv_ckpt_forward_ws_bytes(B, T, C)))) return st;
    const linrec::WkvArgs A{w, u, k, v, y, env_int("LINREC_WKV_EXACT", 0) > 0 ? 1 : 0, r, s_in, s_out};
    // Coordination in wave 0 by default (measured faster); LINREC_COORD=2 gives it a wave of
    // its own.
    const bool sep = env_int("LINREC_COORD", 0) == 2;
    return hip_status(linrec::run_wkv_forward_ckpt(A, B, T, C, ckpt, workspace, next_tag(), spin_limit(), sep,
                                                   (hipStream_t)stream),
                      "wkv4_forward_ckpt launch");
}

LINREC_API int wkv4_forward_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                                 const float* k, const float* v, const float* r, float* y, void* ckpt,
                                 size_t ckpt_bytes, void* workspace, size_t ws_bytes, void* stream) {
    return wkv4_forward_ckpt_ex(B, T, C, w, u, k, v, r, nullptr, y, nullptr, ckpt, ckpt_bytes, workspace, ws_bytes,
                                stream);
}

LINREC_API int wkv4_backward_ckpt_ex(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                                     const float* k, const float* v, const float* r, const float* s_in,
                                     const float* s_out, const float* gy, const float* gs_out, const void* ckpt,
                                     size_t ckpt_bytes, float* gw, float* gu, float* gk, float* gv, float* gr,
                                     float* gs_in, void* workspace, size_t ws_bytes, void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (!r != !gr) return fail(LINREC_ERR_INVALID_ARG, "r and gr must be given together");
    if (C > 0 && (!gw || !gu)) return fail(LINREC_ERR_INVALID_ARG, "gw or gu is NULL");
    if (gs_out && !s_out) return fail(LINREC_ERR_INVALID_ARG, "gs_out needs s_out (its exponents)");
    const void* sptrs[] = {s_in, s_out, gs_out, gs_in};
    for (const void* p : sptrs)
        if (p && !aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "state pointer not 4-byte aligned");
    const linrec::WkvBwdArgs A{w, u, k, v, gy, gw, gu, gk, gv, r, gr, s_in, s_out, gs_out, gs_in};
    if (B == 0 || T == 0 || C == 0) {
        // As wkv4_backward_ex: zero sums, and without tokens the state's gradient passes through.
        if (C == 0) return ok();
        if (!aligned(gw, 4) || !aligned(gu, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
        hipError_t e = linrec::run_zero_wu(gw, gu, C, (hipStream_t)stream);
        if (e == hipSuccess && gs_in && B > 0) e = linrec::run_state_grad_passthrough(A, B, C, (hipStream_t)stream);
        return hip_status(e, "wkv4_backward_ckpt zero-fill");
    }
    if (!w || !u || !k || !v || !gy || !gk || !gv)
        return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {w, u, k, v, gy, gw, gu, gk, gv, r, gr};
    for (const void* p : ptrs)
        if (p && !aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    if ((st = check_ckpt(ckpt, ckpt_bytes, linrec::wkv_ckpt_bytes(B, T, C)))) return st;
    const linrec::BwdPlan p = linrec::wkv_backward_plan(1, B, T, C, 0, 0);  // the checkpoints' slabs
    if ((st = check_ws(workspace, ws_bytes, linrec::wkv_backward_ckpt_ws_bytes(B, T, C)))) return st;
    linrec::BwdGeom g{};
    g.B = B;
    g.T = T;
    g.C = C;
    g.ngrp = ceil_div(C, 64);
    g.nslab = p.nslab;
    g.spin = spin_limit();
    g.tag_f = next_tag();
    g.tag_r = next_tag();
    g.exact_only = env_int("LINREC_WKV_EXACT", 0) > 0 ? 1 : 0;
    linrec::wkv_backward_layout_ckpt(p, B, C, workspace, ckpt, g);
    return hip_status(linrec::run_wkv_backward(A, g, p, (hipStream_t)stream), "wkv4_backward_ckpt launch");
}

LINREC_API int wkv4_backward_ckpt(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                                  const float* k, const float* v, const float* r, const float* gy,
                                  const void* ckpt, size_t ckpt_bytes, float* gw, float* gu, float* gk,
                                  float* gv, float* gr, void* workspace, size_t ws_bytes, void* stream) {
    return wkv4_backward_ckpt_ex(B, T, C, w, u, k, v, r, nullptr, nullptr, gy, nullptr, ckpt, ckpt_bytes, gw, gu, gk,
                                 gv, gr, nullptr, workspace, ws_bytes, stream);
}

LINREC_API int wkv4_backward(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                             const float* k, const float* v, const float* gy, float* gw, float* gu,
                             float* gk, float* gv, void* workspace, size_t ws_bytes, void* stream) {
    return wkv4_backward_ex(B, T, C, w, u, k, v, nullptr, nullptr, nullptr, gy, nullptr, gw, gu, gk, gv, nullptr,
                            nullptr, workspace, ws_bytes, stream);
}

// ---- the forward for callers that cannot allocate ----
// wkv4_forward_noalloc runs wkv4_forward's kernels with their look-back flags and records in
// `scratch`, a file-scope device array, instead of a caller workspace.  The runtime gives
// each GPU its own copy of the array, at its own address: the host-side name is only a
// stand-in, so kernels are handed the address hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.
namespace {

static_assert(LINREC_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch is whole 256-byte blocks");
__device__ __align__(256) unsigned char scratch[LINREC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

// The device address of `scratch` on the current device; the first call on a device looks
// it up (with that device current) and keeps it.
int scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(LINREC_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(LINREC_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return LINREC_OK;
}

}  // namespace

LINREC_API int wkv4_forward_noalloc(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                                    const float* k, const float* v, float* y, void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (B == 0 || T == 0 || C == 0) return ok();
    if (!w || !u || !k || !v || !y) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {w, u, k, v, y};
    for (const void* p : ptrs)
        if (!aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    const int vec = pick_vec(linrec::kKindWkv,
                             (C % 4 == 0 && aligned(k, 16) && aligned(v, 16) && aligned(y, 16))  ? 4
                             : (C % 2 == 0 && aligned(k, 8) && aligned(v, 8) && aligned(y, 8)) ? 2
                                                                                                  : 1,
                             B * T * C, true);
    const linrec::ScanPlan p = scan_plan(linrec::kKindWkv, vec, B, T, C);
    if (p.ws_bytes > (size_t)LINREC_NOALLOC_SCRATCH_BYTES)
        return fail(LINREC_ERR_UNSUPPORTED,
                    "B=%lld T=%lld C=%lld needs %zu bytes of scratch; the static array holds %zu (use wkv4_forward "
                    "with a workspace)",
                    (long long)B, (long long)T, (long long)C, p.ws_bytes, (size_t)LINREC_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws))) return st;
    // The flags carry a per-call tag and the array starts zeroed (static storage), so neither
    // an earlier call's records nor the initial contents read as published: nothing needs
    // clearing.
    const linrec::WkvArgs A{w, u, k, v, y, env_int("LINREC_WKV_EXACT", 0) > 0 ? 1 : 0, nullptr, nullptr, nullptr};
    return hip_status(linrec::run_wkv_forward(A, geom_of(linrec::kKindWkv, p, B, T, C, ws), p, (hipStream_t)stream),
                      "wkv4_forward_noalloc launch");
}
