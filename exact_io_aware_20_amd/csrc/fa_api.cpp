// C ABI of libfa_mi355x.so: argument validation and dispatch to the launchers.
// Every check runs on the host before anything is enqueued.
#include "../../include/fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_launch.hpp"

namespace {

constexpr long long kMaxGrid = 0x7fffffffLL;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

fa_status check_shape(int B, int Hq, int Hkv, int N, int d, int causal, float scale) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_GQA;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (causal != 0 && causal != 1) return FA_ERR_FLAG;
    if (!isfinite(scale) || !(scale >= 0.f)) return FA_ERR_SCALE;
    return FA_OK;
}

// Ranges of the forward's tensors; outputs (o, lse) must not overlap anything.
fa_status check_fwd(const void* q, const void* k, const void* v, const void* o, const void* lse,
                    int B, int Hq, int Hkv, int N, int d, int causal, float scale, int elt) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    fa_status s = check_shape(B, Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    const long long grid = elt == 2 ? fa::fwd_bf16_grid(B, Hq, N, d) : fa::fwd_f32_grid(B, Hq, N);
    if (grid > kMaxGrid) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_ALIGN;
    const uintptr_t qb = (uintptr_t)B * Hq * N * d * elt, kb = (uintptr_t)B * Hkv * N * d * elt;
    const uintptr_t lb = (uintptr_t)B * Hq * N * 4;
    const Range rq{(uintptr_t)q, (uintptr_t)q + qb}, rk{(uintptr_t)k, (uintptr_t)k + kb},
        rv{(uintptr_t)v, (uintptr_t)v + kb}, ro{(uintptr_t)o, (uintptr_t)o + qb},
        rl{(uintptr_t)lse, (uintptr_t)lse + lb};
    const Range outs[2] = {ro, rl};
    const Range ins[3] = {rq, rk, rv};
    for (const Range& a : outs)
        for (const Range& b : ins)
            if (overlap(a, b)) return FA_ERR_ALIAS;
    if (overlap(ro, rl)) return FA_ERR_ALIAS;
    return FA_OK;
}

fa::FwdParams fwd_params(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int Hq, int Hkv, int N, int causal, float scale) {
    fa::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.causal = causal;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    return p;
}

}  // namespace

extern "C" {

fa_status fa_check_args(const void* q, const void* k, const void* v, const void* o, const void* lse,
                        int B, int Hq, int Hkv, int N, int d, int causal, float scale, int elt_bytes) {
    if (elt_bytes != 2 && elt_bytes != 4) return FA_ERR_SHAPE;
    return check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, elt_bytes);
}

fa_status fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                     int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    fa_status s = fa_check_args(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, 2);
    if (s != FA_OK) return s;
    const fa::FwdParams p = fwd_params(q, k, v, o, lse, B, Hq, Hkv, N, causal, scale);
    return fa::launch_fwd_bf16(p, d, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                         int Hq, int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    fa_status s = fa_check_args(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, 4);
    if (s != FA_OK) return s;
    const fa::FwdParams p = fwd_params(q, k, v, o, lse, B, Hq, Hkv, N, causal, scale);
    return fa::launch_fwd_f32(p, d, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_backward_workspace_bytes(int B, int Hq, int N) {
    if (B < 1 || Hq < 1 || N < 1) return 0;
    return (size_t)B * Hq * N * sizeof(float);
}

fa_status fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv, void* workspace,
                      size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, int causal,
                      float scale, hipStream_t stream) {
    if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
    fa_status s = check_shape(B, Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    if (fa::bwd_grid_max(B, Hq, Hkv, N, d) > kMaxGrid) return FA_ERR_SHAPE;
    const void* ptrs[9] = {q, k, v, o, dO, lse, dq, dk, dv};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return FA_ERR_ALIGN;
    const size_t ws_need = fa_backward_workspace_bytes(B, Hq, N);
    if (!workspace || !aligned16(workspace) || workspace_bytes < ws_need) return FA_ERR_WORKSPACE;

    const uintptr_t qb = (uintptr_t)B * Hq * N * d * 2, kb = (uintptr_t)B * Hkv * N * d * 2;
    const uintptr_t lb = (uintptr_t)B * Hq * N * 4;
    const Range ins[6] = {{(uintptr_t)q, (uintptr_t)q + qb},   {(uintptr_t)k, (uintptr_t)k + kb},
                          {(uintptr_t)v, (uintptr_t)v + kb},   {(uintptr_t)o, (uintptr_t)o + qb},
                          {(uintptr_t)dO, (uintptr_t)dO + qb}, {(uintptr_t)lse, (uintptr_t)lse + lb}};
    const Range outs[4] = {{(uintptr_t)dq, (uintptr_t)dq + qb},
                           {(uintptr_t)dk, (uintptr_t)dk + kb},
                           {(uintptr_t)dv, (uintptr_t)dv + kb},
                           {(uintptr_t)workspace, (uintptr_t)workspace + ws_need}};
    for (int i = 0; i < 4; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_ALIAS;
    }

    fa::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dO = dO;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dsum = (float*)workspace;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.causal = causal;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    return fa::launch_bwd_bf16(p, d, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* fa_status_string(fa_status status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "invalid shape: B, Hq, Hkv and N must be >= 1 and the grid must fit";
        case FA_ERR_GQA: return "Hq must be a multiple of Hkv";
        case FA_ERR_HEADDIM: return "head dimension d must be 64 or 128";
        case FA_ERR_SCALE: return "scale must be finite and >= 0";
        case FA_ERR_ALIGN: return "every pointer must be 16-byte aligned";
        case FA_ERR_FLAG: return "causal must be 0 or 1";
        case FA_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than fa_backward_workspace_bytes";
        case FA_ERR_ALIAS: return "an output overlaps an input or another output";
        case FA_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

}  // extern "C"
