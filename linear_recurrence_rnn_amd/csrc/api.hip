// api.hip -- the C ABI declared in include/linrec.h: argument checks, launch plans and
// kernel dispatch.  Host code only; every check runs before any HIP call.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "linrec.h"
#include "chunk_scan.hpp"
#include "wkv_backward.hpp"

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

// Launch plan of the chunked scan; a pure function of (kind, B, T, C) and the
// environment overrides, so the workspace query and the call always agree.
linrec::ScanPlan scan_plan(int kind, int64_t B, int64_t T, int64_t C) {
    linrec::ScanPlan p{};
    p.vec = 1;
    p.rows = (int)env_int("LINREC_ROWS", T >= 512 ? 64 : 16);
    if (p.rows != 16 && p.rows != 64) p.rows = 64;
    const int64_t tile = (int64_t)p.rows * linrec::kChunkLen;
    const int64_t ngrp = ceil_div(C, linrec::kGroupChannels);
    const int64_t wgs = B * ngrp;
    const int64_t max_slabs = T > 0 ? ceil_div(T, tile) : 1;
    int64_t nslab = 1;
    const int64_t forced = env_int("LINREC_NSLAB", 0);
    if (forced > 0) {
        nslab = forced;
    } else if (wgs > 0 && wgs < 512) {
        nslab = ceil_div(1024, wgs);  // aim at ~1024 workgroups on 256 CUs
    }
    if (nslab > max_slabs) nslab = max_slabs;
    if (nslab < 1) nslab = 1;
    p.slab_len = ceil_div(ceil_div(T > 0 ? T : 1, nslab), tile) * tile;
    p.nslab = T > 0 ? ceil_div(T, p.slab_len) : 1;
    p.ws_bytes = 0;
    if (p.nslab > 1) p.ws_bytes = 2 * align256((size_t)(B * p.nslab * C) * linrec::agg_bytes(kind));
    return p;
}

linrec::ScanGeom geom_of(const linrec::ScanPlan& p, int64_t B, int64_t T, int64_t C, void* ws) {
    linrec::ScanGeom g{};
    g.B = B;
    g.T = T;
    g.C = C;
    g.ngrp = ceil_div(C, linrec::kGroupChannels);
    g.nslab = p.nslab;
    g.slab_len = p.slab_len;
    g.mode = linrec::kModeFull;
    g.ws_agg = ws;
    g.ws_carry = p.nslab > 1 ? (char*)ws + p.ws_bytes / 2 : nullptr;
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
    return scan_plan(linrec::kKindWkv, B, T, C).ws_bytes;
}

LINREC_API size_t linrec_scan_workspace_size(int64_t B, int64_t T, int64_t C, int is_complex) {
    if (B < 0 || T < 0 || C < 0 || B == 0 || T == 0 || C == 0) return 0;
    return scan_plan(is_complex ? linrec::kKindComplex : linrec::kKindReal, B, T, C).ws_bytes;
}

LINREC_API size_t wkv4_backward_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || B == 0 || T == 0 || C == 0) return 0;
    return linrec::wkv_backward_plan(B, T, C).ws_bytes;
}

LINREC_API int wkv4_forward(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                            const float* k, const float* v, float* y, void* workspace,
                            size_t ws_bytes, void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (B == 0 || T == 0 || C == 0) return ok();
    if (!w || !u || !k || !v || !y) return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {w, u, k, v, y};
    for (const void* p : ptrs)
        if (!aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    linrec::ScanPlan p = scan_plan(linrec::kKindWkv, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    p.vec = (C % 4 == 0 && aligned(k, 16) && aligned(v, 16) && aligned(y, 16)) ? 4 : 1;
    const linrec::WkvArgs A{w, u, k, v, y, env_int("LINREC_WKV_EXACT", 0) > 0 ? 1 : 0};
    return hip_status(linrec::run_wkv_forward(A, geom_of(p, B, T, C, workspace), p, (hipStream_t)stream),
                      "wkv4_forward launch");
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
    linrec::ScanPlan p = scan_plan(linrec::kKindReal, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    p.vec = (C % 4 == 0 && aligned(a, 16) && aligned(b, 16) && aligned(x, 16)) ? 4 : 1;
    const linrec::RealArgs A{a, b, x0, x};
    return hip_status(linrec::run_scan_real(A, geom_of(p, B, T, C, workspace), p, (hipStream_t)stream),
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
    linrec::ScanPlan p = scan_plan(linrec::kKindComplex, B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    p.vec = (C % 2 == 0 && aligned(u, 16) && aligned(x, 16)) ? 2 : 1;
    const linrec::CplxArgs A{lambda, u, x0, x};
    return hip_status(linrec::run_scan_complex(A, geom_of(p, B, T, C, workspace), p, (hipStream_t)stream),
                      "linrec_scan_complex launch");
}

LINREC_API int wkv4_backward(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                             const float* k, const float* v, const float* gy, float* gw, float* gu,
                             float* gk, float* gv, void* workspace, size_t ws_bytes, void* stream) {
    int st = check_shape(B, T, C, 4);
    if (st) return st;
    if (C > 0 && (!gw || !gu)) return fail(LINREC_ERR_INVALID_ARG, "gw or gu is NULL");
    if (B == 0 || T == 0 || C == 0) {
        // Empty batch or sequence: the per-channel sums dL/dw, dL/du are zero.
        if (C == 0) return ok();
        if (!aligned(gw, 4) || !aligned(gu, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
        return hip_status(linrec::run_zero_wu(gw, gu, C, (hipStream_t)stream), "wkv4_backward zero-fill");
    }
    if (!w || !u || !k || !v || !gy || !gk || !gv)
        return fail(LINREC_ERR_INVALID_ARG, "a required pointer is NULL");
    const void* ptrs[] = {w, u, k, v, gy, gw, gu, gk, gv};
    for (const void* p : ptrs)
        if (!aligned(p, 4)) return fail(LINREC_ERR_UNSUPPORTED, "pointer not 4-byte aligned");
    linrec::BwdPlan p = linrec::wkv_backward_plan(B, T, C);
    if ((st = check_ws(workspace, ws_bytes, p.ws_bytes))) return st;
    p.vec = (C % 2 == 0 && aligned(k, 8) && aligned(v, 8) && aligned(gy, 8) && aligned(gk, 8) &&
             aligned(gv, 8))
                ? 2
                : 1;
    const linrec::WkvBwdArgs A{w, u, k, v, gy, gw, gu, gk, gv};
    return hip_status(linrec::run_wkv_backward(A, B, T, C, p, workspace, (hipStream_t)stream),
                      "wkv4_backward launch");
}
