// C ABI of libfa_mi355x.so: argument validation and dispatch to the launchers.
// Every check runs on the host before anything is enqueued.
#include "../../include/fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_launch.hpp"

namespace {

constexpr long long kMaxGrid = 0x7fffffffLL;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Backward workspace, by query row r of R = B*Hq*N:
//   [0, 8R)                D_r (fp32), then LSE_r * log2(e) (fp32): all that fa_backward
//                          and its dK/dV and dQ kernels use;
//   [align256(8R), + 4dR)  the fused alternative's fp32 dQ accumulator [R][d] (zeroed
//                          by the preprocess when the workspace has room for it, added
//                          to by the fused kernel, read by the conversion to bf16).
size_t bwd_ws_bytes(int B, int Hq, int N) {
    if (B < 1 || Hq < 1 || N < 1) return 0;
    return (size_t)B * Hq * N * 2 * sizeof(float);
}
size_t bwd_dqacc_offset(int B, int Hq, int N) { return (bwd_ws_bytes(B, Hq, N) + 255) & ~(size_t)255; }
size_t bwd_fused_ws_bytes(int B, int Hq, int N, int d) {
    if (B < 1 || Hq < 1 || N < 1 || (d != 64 && d != 128)) return 0;
    return bwd_dqacc_offset(B, Hq, N) + (size_t)B * Hq * N * d * sizeof(float);
}

fa_status check_shape(int B, int Hq, int Hkv, int N, int d, int causal, float scale) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_GQA;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (causal != 0 && causal != 1) return FA_ERR_FLAG;
    if (!isfinite(scale) || !(scale >= 0.f)) return FA_ERR_SCALE;
    return FA_OK;
}

// One tensor argument: address, byte size, written (output) or only read.
struct Arg {
    const void* ptr;
    uintptr_t bytes;
    bool out;
};

// Null, alignment and overlap checks; an output may overlap no other argument.
fa_status check_tensors(const Arg* a, int n) {
    for (int i = 0; i < n; ++i)
        if (!a[i].ptr) return FA_ERR_NULL;
    for (int i = 0; i < n; ++i)
        if (!aligned16(a[i].ptr)) return FA_ERR_ALIGN;
    for (int i = 0; i < n; ++i) {
        if (!a[i].out) continue;
        const uintptr_t lo = (uintptr_t)a[i].ptr, hi = lo + a[i].bytes;
        for (int j = 0; j < n; ++j) {
            if (j == i) continue;
            const uintptr_t lo2 = (uintptr_t)a[j].ptr, hi2 = lo2 + a[j].bytes;
            if (lo < hi2 && lo2 < hi) return FA_ERR_ALIAS;
        }
    }
    return FA_OK;
}

fa_status check_fwd(const void* q, const void* k, const void* v, const void* o, const void* lse, int B,
                    int Hq, int Hkv, int N, int d, int causal, float scale, int elt) {
    if (elt != 2 && elt != 4) return FA_ERR_SHAPE;
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    fa_status s = check_shape(B, Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    const long long grid = elt == 2 ? fa::fwd_bf16_grid(B, Hq, N, d) : fa::fwd_f32_grid(B, Hq, N);
    if (grid > kMaxGrid) return FA_ERR_SHAPE;
    const uintptr_t qb = (uintptr_t)B * Hq * N * d * elt, kb = (uintptr_t)B * Hkv * N * d * elt;
    const Arg a[5] = {{q, qb, false}, {k, kb, false}, {v, kb, false}, {o, qb, true},
                      {lse, (uintptr_t)B * Hq * N * 4, true}};
    return check_tensors(a, 5);
}

// kAll: a whole backward call; kPre: the preprocess; kDkdv, kDq: the two kernels of the
// deterministic pair (they read only the small workspace); kPreDq: the dQ kernel that
// forms the per-row terms itself and writes them to the workspace; kFused: the fused
// dK/dV/dQ kernel (adds into the dQ accumulator); kConvert: accumulator -> dq.
enum BwdStep { kAll, kPre, kDkdv, kDq, kPreDq, kFused, kConvert };

fa_status check_bwd(BwdStep step, const void* q, const void* k, const void* v, const void* o,
                    const void* dO, const void* lse, const void* dq, const void* dk, const void* dv,
                    const void* workspace, size_t ws_bytes, int B, int Hq, int Hkv, int N, int d,
                    int causal, float scale) {
    fa_status s = check_shape(B, Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    if (fa::bwd_grid_max(B, Hq, Hkv, N, d) > kMaxGrid) return FA_ERR_SHAPE;
    const bool fused = step == kFused || step == kConvert;
    const size_t ws_need = fused ? bwd_fused_ws_bytes(B, Hq, N, d) : bwd_ws_bytes(B, Hq, N);
    if (!workspace || !aligned16(workspace) || ws_bytes < ws_need) return FA_ERR_WORKSPACE;
    const uintptr_t qb = (uintptr_t)B * Hq * N * d * 2, kb = (uintptr_t)B * Hkv * N * d * 2;
    const uintptr_t lb = (uintptr_t)B * Hq * N * 4;
    Arg a[11];
    int n = 0;
    // the preprocess also zeroes the fused accumulator when the workspace has room for it
    const size_t fused_need = bwd_fused_ws_bytes(B, Hq, N, d);
    const size_t ws_extent = step == kPre && ws_bytes >= fused_need ? fused_need : ws_need;
    a[n++] = {workspace, ws_extent, step == kAll || step == kPre || step == kPreDq || step == kFused};
    if (step != kConvert) a[n++] = {dO, qb, false};
    if (step == kAll || step == kPre || step == kPreDq) {
        a[n++] = {o, qb, false};
        a[n++] = {lse, lb, false};
    }
    if (step != kPre && step != kConvert) {
        a[n++] = {q, qb, false};
        a[n++] = {k, kb, false};
        a[n++] = {v, kb, false};
    }
    if (step == kAll || step == kDq || step == kPreDq || step == kConvert) a[n++] = {dq, qb, true};
    if (step == kAll || step == kDkdv || step == kFused) {
        a[n++] = {dk, kb, true};
        a[n++] = {dv, kb, true};
    }
    return check_tensors(a, n);
}

// scale * log2(e) as the kernels use it.  The kernels mask a score by setting it
// to -inf and rely on -inf * scale_log2 = -inf (p = exp2(-inf) = 0); for scale = 0
// the smallest normal float is used instead: any score below 2^60 in magnitude
// times it is below 2^-66, so exp2 of it rounds to exactly 1.0, as exp(0 * s) is;
// LSE and the gradients (which use `scale` itself) are unchanged.
float kernel_scale_log2(float scale) {
    const float s = scale * 1.4426950408889634f;
    return s > 0.f ? s : 1.17549435e-38f;
}

fa_status check_decode_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale) {
    fa_status s = check_shape(B, Hq, Hkv, Nk, d, causal, scale);
    if (s != FA_OK) return s;
    if (Nq < 1 || (causal && Nq > Nk)) return FA_ERR_SHAPE;
    if (fa::decode_plan(B, Hq, Hkv, Nq, Nk, d).grid > kMaxGrid || (long long)B * Hq * Nq > kMaxGrid)
        return FA_ERR_SHAPE;
    return FA_OK;
}

fa_status check_decode(const void* q, const void* k, const void* v, const void* o, const void* lse,
                       const void* workspace, size_t ws_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                       int causal, float scale) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    fa_status s = check_decode_shape(B, Hq, Hkv, Nq, Nk, d, causal, scale);
    if (s != FA_OK) return s;
    const size_t ws_need = fa::decode_plan(B, Hq, Hkv, Nq, Nk, d).workspace_bytes;
    if (!workspace || !aligned16(workspace) || ws_bytes < ws_need) return FA_ERR_WORKSPACE;
    const uintptr_t qb = (uintptr_t)B * Hq * Nq * d * 2, kb = (uintptr_t)B * Hkv * Nk * d * 2;
    const Arg a[6] = {{q, qb, false}, {k, kb, false}, {v, kb, false}, {o, qb, true},
                      {lse, (uintptr_t)B * Hq * Nq * 4, true}, {workspace, ws_need, true}};
    return check_tensors(a, 6);
}

fa::FwdParams fwd_params(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                         int Hkv, int N, int causal, float scale) {
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
    p.window = -1;
    p.block_mask = nullptr;
    p.scale = scale;
    p.scale_log2 = kernel_scale_log2(scale);
    p.o32 = nullptr;
    return p;
}

fa::BwdParams bwd_params(const void* q, const void* k, const void* v, const void* o, const void* dO,
                         const float* lse, void* dq, void* dk, void* dv, const void* workspace, int B,
                         int Hq, int Hkv, int N, int causal, float scale) {
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
    p.lse2 = (float*)workspace + (size_t)B * Hq * N;
    p.dqacc = nullptr;   // set by the calls of the fused alternative
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.causal = causal;
    p.window = -1;
    p.block_mask = nullptr;
    p.scale = scale;
    p.scale_log2 = kernel_scale_log2(scale);
    p.form_rows = 0;
    return p;
}

// A window as wide as the sequence restricts nothing: the kernels take it as none.
int kernel_window(int window, int N) { return window < N - 1 ? window : -1; }

fa_status launched(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

// The backward as fa_backward runs it: the dQ kernel, which forms the per-row terms (D,
// LSE in base 2) itself, bit for bit as the preprocess does, and writes them to the
// workspace; then the dK/dV kernel, which reads them.  Under a block-sparse layout the
// preprocess runs on its own first, then dK/dV, then dQ: there the light dK/dV kernel
// measured 5 % slower after the dQ kernel than after the preprocess's pass over O and dO.
fa_status pair_backward(const fa::BwdParams& p, int d, hipStream_t stream) {
    fa_status s;
    if (p.block_mask) {
        if ((s = launched(fa::launch_bwd_pre(p, d, stream))) != FA_OK) return s;
        if ((s = launched(fa::launch_bwd_dkdv(p, d, stream))) != FA_OK) return s;
        return launched(fa::launch_bwd_dq(p, d, stream));
    }
    if ((s = launched(fa::launch_bwd_dq_rows(p, d, stream))) != FA_OK) return s;
    return launched(fa::launch_bwd_dkdv(p, d, stream));
}

// The fused alternative: the workspace's dQ accumulator follows the per-row terms.
void set_fused_accumulator(fa::BwdParams& p, const void* workspace, int B, int Hq, int N) {
    p.dqacc = (float*)((const char*)workspace + bwd_dqacc_offset(B, Hq, N));
}

}  // namespace

extern "C" {

fa_status fa_check_args(const void* q, const void* k, const void* v, const void* o, const void* lse, int B,
                        int Hq, int Hkv, int N, int d, int causal, float scale, int elt_bytes) {
    return check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, elt_bytes);
}

fa_status fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                     int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    fa_status s = check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, 2);
    if (s != FA_OK) return s;
    return launched(fa::launch_fwd_bf16(fwd_params(q, k, v, o, lse, B, Hq, Hkv, N, causal, scale), d, stream));
}

fa_status fa_forward_fp32_out(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
                              int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    // o holds fp32 elements: validated as a 4-byte output against bf16 inputs
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    fa_status s = check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, 2);
    if (s != FA_OK) return s;
    const uintptr_t ob = (uintptr_t)B * Hq * N * d * 4, kb = (uintptr_t)B * Hkv * N * d * 2;
    const Arg a[5] = {{q, (uintptr_t)B * Hq * N * d * 2, false}, {k, kb, false}, {v, kb, false}, {o, ob, true},
                      {lse, (uintptr_t)B * Hq * N * 4, true}};
    if ((s = check_tensors(a, 5)) != FA_OK) return s;
    fa::FwdParams p = fwd_params(q, k, v, nullptr, lse, B, Hq, Hkv, N, causal, scale);
    p.o32 = o;
    return launched(fa::launch_fwd_bf16(p, d, stream));
}

fa_status fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                         int Hq, int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    fa_status s = check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, 4);
    if (s != FA_OK) return s;
    return launched(fa::launch_fwd_f32(fwd_params(q, k, v, o, lse, B, Hq, Hkv, N, causal, scale), d, stream));
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    if (check_decode_shape(B, Hq, Hkv, Nq, Nk, d, 0, 1.f) != FA_OK) return 0;
    return fa::decode_plan(B, Hq, Hkv, Nq, Nk, d).workspace_bytes;
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

fa_status check_paged(const void* q, const void* kp, const void* vp, const int* table, const int* seq_lens,
                      const void* o, const void* lse, const void* workspace, size_t ws_bytes, int B, int Hq, int Hkv,
                      int Nq, int max_seq_len, int num_pages, int page_size, int max_blocks, int d, int causal,
                      float scale) {
    if (!q || !kp || !vp || !table || !seq_lens || !o || !lse) return FA_ERR_NULL;
    fa_status s = check_decode_shape(B, Hq, Hkv, Nq, max_seq_len, d, causal, scale);
    if (s != FA_OK) return s;
    if (page_size < 64 || page_size % 64 != 0 || max_blocks < 1 || num_pages < 1 ||
        (long long)max_blocks * page_size < max_seq_len)
        return FA_ERR_SHAPE;
    const size_t ws_need = fa::decode_plan(B, Hq, Hkv, Nq, max_seq_len, d).workspace_bytes;
    if (!workspace || !aligned16(workspace) || ws_bytes < ws_need) return FA_ERR_WORKSPACE;
    if (!aligned4(table) || !aligned4(seq_lens)) return FA_ERR_ALIGN;
    const uintptr_t qb = (uintptr_t)B * Hq * Nq * d * 2;
    const uintptr_t pb = (uintptr_t)num_pages * Hkv * page_size * d * 2;
    const Arg a[8] = {{q, qb, false},
                      {kp, pb, false},
                      {vp, pb, false},
                      {table, (uintptr_t)B * max_blocks * 4, false},
                      {seq_lens, (uintptr_t)B * 4, false},
                      {o, qb, true},
                      {lse, (uintptr_t)B * Hq * Nq * 4, true},
                      {workspace, ws_need, true}};
    // the table and lengths (entries 3, 4) need only 4-byte alignment; every entry is
    // checked for overlap with the outputs
    for (int i = 0; i < 8; ++i)
        if (i != 3 && i != 4 && !aligned16(a[i].ptr)) return FA_ERR_ALIGN;
    for (int i = 0; i < 8; ++i) {
        if (!a[i].out) continue;
        const uintptr_t lo = (uintptr_t)a[i].ptr, hi = lo + a[i].bytes;
        for (int j = 0; j < 8; ++j) {
            if (j == i) continue;
            const uintptr_t lo2 = (uintptr_t)a[j].ptr, hi2 = lo2 + a[j].bytes;
            if (lo < hi2 && lo2 < hi) return FA_ERR_ALIAS;
        }
    }
    return FA_OK;
}

static fa_status decode_call(int steps, const void* q, const void* k, const void* v, void* o, float* lse,
                             void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk,
                             int d, int causal, float scale, hipStream_t stream) {
    fa_status s = check_decode(q, k, v, o, lse, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d, causal, scale);
    if (s != FA_OK) return s;
    const fa::DecodePlan pl = fa::decode_plan(B, Hq, Hkv, Nq, Nk, d);
    fa::DecodeParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.part_o = (float*)workspace;
    p.part_lse = (float*)workspace + (size_t)pl.nsplit * B * Hq * Nq * d;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = Nq;
    p.Nk = Nk;
    p.causal = causal;
    p.nrb = pl.nrb;
    p.nsplit = pl.nsplit;
    p.tiles_per_split = pl.tiles_per_split;
    p.scale_log2 = kernel_scale_log2(scale);
    p.block_table = nullptr;
    p.seq_lens = nullptr;
    p.max_blocks = p.page_size = p.num_pages = 0;
    return launched(fa::launch_decode(p, d, steps, false, stream));
}

static fa_status paged_call(int steps, const void* q, const void* kp, const void* vp, const int* table,
                            const int* seq_lens, void* o, float* lse, void* workspace, size_t workspace_bytes, int B,
                            int Hq, int Hkv, int Nq, int max_seq_len, int num_pages, int page_size, int max_blocks,
                            int d, int causal, float scale, hipStream_t stream) {
    fa_status s = check_paged(q, kp, vp, table, seq_lens, o, lse, workspace, workspace_bytes, B, Hq, Hkv, Nq,
                              max_seq_len, num_pages, page_size, max_blocks, d, causal, scale);
    if (s != FA_OK) return s;
    const fa::DecodePlan pl = fa::decode_plan(B, Hq, Hkv, Nq, max_seq_len, d);
    fa::DecodeParams p;
    p.q = q;
    p.k = kp;
    p.v = vp;
    p.o = o;
    p.lse = lse;
    p.part_o = (float*)workspace;
    p.part_lse = (float*)workspace + (size_t)pl.nsplit * B * Hq * Nq * d;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = Nq;
    p.Nk = max_seq_len;
    p.causal = causal;
    p.block_table = table;
    p.seq_lens = seq_lens;
    p.max_blocks = max_blocks;
    p.page_size = page_size;
    p.num_pages = num_pages;
    p.nrb = pl.nrb;
    p.nsplit = pl.nsplit;
    p.tiles_per_split = pl.tiles_per_split;
    p.scale_log2 = kernel_scale_log2(scale);
    return launched(fa::launch_decode(p, d, steps, true, stream));
}

fa_status fa_decode_forward(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                            size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                            float scale, hipStream_t stream) {
    return decode_call(fa::kDecodeSplit | fa::kDecodeMerge, q, k, v, o, lse, workspace, workspace_bytes, B, Hq,
                       Hkv, Nq, Nk, d, causal, scale, stream);
}

fa_status fa_decode_split(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                          size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, hipStream_t stream) {
    return decode_call(fa::kDecodeSplit, q, k, v, o, lse, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d,
                       causal, scale, stream);
}

fa_status fa_decode_merge(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                          size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, hipStream_t stream) {
    return decode_call(fa::kDecodeMerge, q, k, v, o, lse, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d,
                       causal, scale, stream);
}

#define FA_PAGED_ARGS                                                                                           \
    const void *q, const void *k_pages, const void *v_pages, const int *block_table, const int *seq_lens, void *o, \
        float *lse, void *workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int max_seq_len,     \
        int num_pages, int page_size, int max_blocks, int d, int causal, float scale, hipStream_t stream
#define FA_PAGED_PASS                                                                                          \
    q, k_pages, v_pages, block_table, seq_lens, o, lse, workspace, workspace_bytes, B, Hq, Hkv, Nq, max_seq_len, \
        num_pages, page_size, max_blocks, d, causal, scale, stream

fa_status fa_decode_paged_forward(FA_PAGED_ARGS) {
    return paged_call(fa::kDecodeSplit | fa::kDecodeMerge, FA_PAGED_PASS);
}
fa_status fa_decode_paged_split(FA_PAGED_ARGS) { return paged_call(fa::kDecodeSplit, FA_PAGED_PASS); }
fa_status fa_decode_paged_merge(FA_PAGED_ARGS) { return paged_call(fa::kDecodeMerge, FA_PAGED_PASS); }

size_t fa_backward_workspace_bytes(int B, int Hq, int N) { return bwd_ws_bytes(B, Hq, N); }

fa_status fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      int B, int Hq, int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    fa_status s = check_bwd(kAll, q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                            N, d, causal, scale);
    if (s != FA_OK) return s;
    const fa::BwdParams p = bwd_params(q, k, v, o, dO, lse, dq, dk, dv, workspace, B, Hq, Hkv, N, causal, scale);
    return pair_backward(p, d, stream);
}

size_t fa_backward_fused_workspace_bytes(int B, int Hq, int N, int d) { return bwd_fused_ws_bytes(B, Hq, N, d); }

fa_status fa_backward_fused(const void* q, const void* k, const void* v, const void* o, const void* dO,
                            const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                            int B, int Hq, int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    fa_status s = check_bwd(kAll, q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, d,
                            causal, scale);
    if (s != FA_OK) return s;
    if (workspace_bytes < bwd_fused_ws_bytes(B, Hq, N, d)) return FA_ERR_WORKSPACE;
    const uintptr_t qb = (uintptr_t)B * Hq * N * d * 2, kb = (uintptr_t)B * Hkv * N * d * 2;
    const Arg a[10] = {{workspace, bwd_fused_ws_bytes(B, Hq, N, d), true}, {q, qb, false}, {k, kb, false},
                       {v, kb, false}, {o, qb, false}, {dO, qb, false}, {lse, (uintptr_t)B * Hq * N * 4, false},
                       {dq, qb, true}, {dk, kb, true}, {dv, kb, true}};
    if ((s = check_tensors(a, 10)) != FA_OK) return s;
    fa::BwdParams p = bwd_params(q, k, v, o, dO, lse, dq, dk, dv, workspace, B, Hq, Hkv, N, causal, scale);
    set_fused_accumulator(p, workspace, B, Hq, N);
    if ((s = launched(fa::launch_bwd_pre(p, d, stream))) != FA_OK) return s;
    if ((s = launched(fa::launch_bwd_fused(p, d, stream))) != FA_OK) return s;
    return launched(fa::launch_bwd_dq_convert(p, d, stream));
}

fa_status fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                              const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                              int causal, float scale, hipStream_t stream) {
    // validated as fa_backward, except that the per-row workspace is the library's own
    // static scratch (which no caller tensor can overlap)
    fa_status s = check_shape(B, Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    if ((long long)B * Hq * N > fa::kScratchRows) return FA_ERR_SCRATCH;
    const uintptr_t qb = (uintptr_t)B * Hq * N * d * 2, kb = (uintptr_t)B * Hkv * N * d * 2;
    const uintptr_t lb = (uintptr_t)B * Hq * N * 4;
    const Arg a[9] = {{q, qb, false}, {k, kb, false}, {v, kb, false}, {o, qb, false}, {dO, qb, false},
                      {lse, lb, false}, {dq, qb, true}, {dk, kb, true}, {dv, kb, true}};
    if ((s = check_tensors(a, 9)) != FA_OK) return s;
    if (fa::bwd_grid_max(B, Hq, Hkv, N, d) > kMaxGrid) return FA_ERR_SHAPE;
    float* ws = nullptr;
    if ((s = launched(fa::bwd_scratch(stream, &ws))) != FA_OK) return s;
    const fa::BwdParams p = bwd_params(q, k, v, o, dO, lse, dq, dk, dv, ws, B, Hq, Hkv, N, causal, scale);
    return pair_backward(p, d, stream);
}

fa_status fa_forward_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                            int Hkv, int N, int d, int causal, int window, float scale, hipStream_t stream) {
    if (window < 0) return FA_ERR_WINDOW;
    fa_status s = check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, 2);
    if (s != FA_OK) return s;
    fa::FwdParams p = fwd_params(q, k, v, o, lse, B, Hq, Hkv, N, causal, scale);
    p.window = kernel_window(window, N);
    return launched(fa::launch_fwd_bf16(p, d, stream));
}

fa_status fa_backward_window(const void* q, const void* k, const void* v, const void* o, const void* dO,
                             const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             int B, int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                             hipStream_t stream) {
    if (window < 0) return FA_ERR_WINDOW;
    fa_status s = check_bwd(kAll, q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                            N, d, causal, scale);
    if (s != FA_OK) return s;
    fa::BwdParams p = bwd_params(q, k, v, o, dO, lse, dq, dk, dv, workspace, B, Hq, Hkv, N, causal, scale);
    p.window = kernel_window(window, N);
    return pair_backward(p, d, stream);
}

fa_status fa_backward_dkdv_window(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
                                  size_t workspace_bytes, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                                  int causal, int window, float scale, hipStream_t stream) {
    if (window < 0) return FA_ERR_WINDOW;
    fa_status s = check_bwd(kDkdv, q, k, v, nullptr, dO, nullptr, nullptr, dk, dv, workspace, workspace_bytes, B,
                            Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    fa::BwdParams p =
        bwd_params(q, k, v, nullptr, dO, nullptr, nullptr, dk, dv, workspace, B, Hq, Hkv, N, causal, scale);
    p.window = kernel_window(window, N);
    return launched(fa::launch_bwd_dkdv(p, d, stream));
}

fa_status fa_backward_dq_window(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
                                size_t workspace_bytes, void* dq, int B, int Hq, int Hkv, int N, int d, int causal,
                                int window, float scale, hipStream_t stream) {
    if (window < 0) return FA_ERR_WINDOW;
    fa_status s = check_bwd(kDq, q, k, v, nullptr, dO, nullptr, dq, nullptr, nullptr, workspace, workspace_bytes, B,
                            Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    fa::BwdParams p =
        bwd_params(q, k, v, nullptr, dO, nullptr, dq, nullptr, nullptr, workspace, B, Hq, Hkv, N, causal, scale);
    p.window = kernel_window(window, N);
    return launched(fa::launch_bwd_dq(p, d, stream));
}

fa_status fa_backward_preprocess_dq_window(const void* q, const void* k, const void* v, const void* o,
                                           const void* dO, const float* lse, void* workspace, size_t workspace_bytes,
                                           void* dq, int B, int Hq, int Hkv, int N, int d, int causal, int window,
                                           float scale, hipStream_t stream) {
    if (window < 0) return FA_ERR_WINDOW;
    fa_status s = check_bwd(kPreDq, q, k, v, o, dO, lse, dq, nullptr, nullptr, workspace, workspace_bytes, B, Hq,
                            Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    fa::BwdParams p = bwd_params(q, k, v, o, dO, lse, dq, nullptr, nullptr, workspace, B, Hq, Hkv, N, causal, scale);
    p.window = kernel_window(window, N);
    return launched(fa::launch_bwd_dq_rows(p, d, stream));
}

// Block-sparse calls: the layout must be present and cover at most 2048 x 2048
// blocks; it is an input of every step, so no output may overlap it.
static fa_status check_layout(const void* block_mask, const void* const* outs, const uintptr_t* out_bytes, int nout,
                       int N) {
    if (!block_mask) return FA_ERR_NULL;
    const long long nb = (N + fa::kSparseBlockHost - 1) / fa::kSparseBlockHost;
    if (nb > fa::kSparseMaxBlocksHost) return FA_ERR_SHAPE;
    const uintptr_t lo = (uintptr_t)block_mask, hi = lo + (uintptr_t)(nb * nb);
    for (int i = 0; i < nout; ++i) {
        const uintptr_t lo2 = (uintptr_t)outs[i], hi2 = lo2 + out_bytes[i];
        if (outs[i] && lo < hi2 && lo2 < hi) return FA_ERR_ALIAS;
    }
    return FA_OK;
}

fa_status fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const unsigned char* block_mask, int B, int Hq, int Hkv, int N, int d, int causal,
                                 float scale, hipStream_t stream) {
    fa_status s = check_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, 2);
    if (s != FA_OK) return s;
    const void* outs[2] = {o, lse};
    const uintptr_t ob[2] = {(uintptr_t)B * Hq * N * d * 2, (uintptr_t)B * Hq * N * 4};
    if ((s = check_layout(block_mask, outs, ob, 2, N)) != FA_OK) return s;
    fa::FwdParams p = fwd_params(q, k, v, o, lse, B, Hq, Hkv, N, causal, scale);
    p.block_mask = block_mask;
    return launched(fa::launch_fwd_bf16(p, d, stream));
}

static fa_status bwd_blocksparse(int steps, const void* q, const void* k, const void* v, const void* o,
                                 const void* dO, const float* lse, void* dq, void* dk, void* dv,
                                 const unsigned char* block_mask, void* workspace, size_t workspace_bytes, int B,
                                 int Hq, int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    // steps: 7 the whole call, 2 the dK/dV step, 4 the dQ step, 5 the dQ step that forms
    // the per-row terms (the preprocess and dQ in one kernel)
    const BwdStep step = steps == 7 ? kAll : (steps == 2 ? kDkdv : (steps == 5 ? kPreDq : kDq));
    fa_status s = check_bwd(step, q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, d,
                            causal, scale);
    if (s != FA_OK) return s;
    const uintptr_t qb = (uintptr_t)B * Hq * N * d * 2, kb = (uintptr_t)B * Hkv * N * d * 2;
    const void* outs[4] = {(steps & 4) ? dq : nullptr, (steps & 2) ? dk : nullptr, (steps & 2) ? dv : nullptr,
                           (steps & 1) ? workspace : nullptr};
    // the workspace's extent is what the call uses (the caller's figure may be any
    // larger value, and adding it to the address could wrap)
    const uintptr_t ob[4] = {qb, kb, kb, (uintptr_t)bwd_ws_bytes(B, Hq, N)};
    if ((s = check_layout(block_mask, outs, ob, 4, N)) != FA_OK) return s;
    fa::BwdParams p = bwd_params(q, k, v, o, dO, lse, dq, dk, dv, workspace, B, Hq, Hkv, N, causal, scale);
    p.block_mask = block_mask;
    if (steps == 7) return pair_backward(p, d, stream);
    if (steps == 2) return launched(fa::launch_bwd_dkdv(p, d, stream));
    if (steps == 5) return launched(fa::launch_bwd_dq_rows(p, d, stream));
    return launched(fa::launch_bwd_dq(p, d, stream));
}

fa_status fa_backward_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                  const float* lse, void* dq, void* dk, void* dv, const unsigned char* block_mask,
                                  void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                                  int causal, float scale, hipStream_t stream) {
    return bwd_blocksparse(7, q, k, v, o, dO, lse, dq, dk, dv, block_mask, workspace, workspace_bytes, B, Hq, Hkv,
                           N, d, causal, scale, stream);
}

fa_status fa_backward_dkdv_blocksparse(const void* q, const void* k, const void* v, const void* dO,
                                       const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                                       const unsigned char* block_mask, int B, int Hq, int Hkv, int N, int d,
                                       int causal, float scale, hipStream_t stream) {
    return bwd_blocksparse(2, q, k, v, nullptr, dO, nullptr, nullptr, dk, dv, block_mask, (void*)workspace,
                           workspace_bytes, B, Hq, Hkv, N, d, causal, scale, stream);
}

fa_status fa_backward_dq_blocksparse(const void* q, const void* k, const void* v, const void* dO,
                                     const void* workspace, size_t workspace_bytes, void* dq,
                                     const unsigned char* block_mask, int B, int Hq, int Hkv, int N, int d,
                                     int causal, float scale, hipStream_t stream) {
    return bwd_blocksparse(4, q, k, v, nullptr, dO, nullptr, dq, nullptr, nullptr, block_mask, (void*)workspace,
                           workspace_bytes, B, Hq, Hkv, N, d, causal, scale, stream);
}

fa_status fa_backward_preprocess_dq_blocksparse(const void* q, const void* k, const void* v, const void* o,
                                                const void* dO, const float* lse, void* workspace,
                                                size_t workspace_bytes, void* dq, const unsigned char* block_mask,
                                                int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                                                hipStream_t stream) {
    return bwd_blocksparse(5, q, k, v, o, dO, lse, dq, nullptr, nullptr, block_mask, workspace, workspace_bytes, B,
                           Hq, Hkv, N, d, causal, scale, stream);
}

fa_status fa_backward_preprocess(const void* o, const void* dO, const float* lse, void* workspace,
                                 size_t workspace_bytes, int B, int Hq, int N, int d, hipStream_t stream) {
    fa_status s = check_bwd(kPre, nullptr, nullptr, nullptr, o, dO, lse, nullptr, nullptr, nullptr,
                            workspace, workspace_bytes, B, Hq, Hq, N, d, 0, 1.f);
    if (s != FA_OK) return s;
    fa::BwdParams p = bwd_params(nullptr, nullptr, nullptr, o, dO, lse, nullptr, nullptr, nullptr,
                                 workspace, B, Hq, Hq, N, 0, 1.f);
    if (workspace_bytes >= bwd_fused_ws_bytes(B, Hq, N, d)) set_fused_accumulator(p, workspace, B, Hq, N);
    return launched(fa::launch_bwd_pre(p, d, stream));
}

fa_status fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
                           size_t workspace_bytes, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                           int causal, float scale, hipStream_t stream) {
    fa_status s = check_bwd(kDkdv, q, k, v, nullptr, dO, nullptr, nullptr, dk, dv, workspace, workspace_bytes, B,
                            Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    const fa::BwdParams p =
        bwd_params(q, k, v, nullptr, dO, nullptr, nullptr, dk, dv, workspace, B, Hq, Hkv, N, causal, scale);
    return launched(fa::launch_bwd_dkdv(p, d, stream));
}

fa_status fa_backward_dq(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
                         size_t workspace_bytes, void* dq, int B, int Hq, int Hkv, int N, int d, int causal,
                         float scale, hipStream_t stream) {
    fa_status s = check_bwd(kDq, q, k, v, nullptr, dO, nullptr, dq, nullptr, nullptr, workspace, workspace_bytes, B,
                            Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    const fa::BwdParams p =
        bwd_params(q, k, v, nullptr, dO, nullptr, dq, nullptr, nullptr, workspace, B, Hq, Hkv, N, causal, scale);
    return launched(fa::launch_bwd_dq(p, d, stream));
}

fa_status fa_backward_preprocess_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                    const float* lse, void* workspace, size_t workspace_bytes, void* dq, int B,
                                    int Hq, int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    fa_status s = check_bwd(kPreDq, q, k, v, o, dO, lse, dq, nullptr, nullptr, workspace, workspace_bytes, B, Hq,
                            Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    const fa::BwdParams p =
        bwd_params(q, k, v, o, dO, lse, dq, nullptr, nullptr, workspace, B, Hq, Hkv, N, causal, scale);
    return launched(fa::launch_bwd_dq_rows(p, d, stream));
}

fa_status fa_backward_dkdv_dq(const void* q, const void* k, const void* v, const void* dO, void* workspace,
                              size_t workspace_bytes, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                              int causal, float scale, hipStream_t stream) {
    fa_status s = check_bwd(kFused, q, k, v, nullptr, dO, nullptr, nullptr, dk, dv, workspace, workspace_bytes, B,
                            Hq, Hkv, N, d, causal, scale);
    if (s != FA_OK) return s;
    fa::BwdParams p =
        bwd_params(q, k, v, nullptr, dO, nullptr, nullptr, dk, dv, workspace, B, Hq, Hkv, N, causal, scale);
    set_fused_accumulator(p, workspace, B, Hq, N);
    return launched(fa::launch_bwd_fused(p, d, stream));
}

fa_status fa_backward_dq_convert(const void* workspace, size_t workspace_bytes, void* dq, int B, int Hq, int N,
                                 int d, float scale, hipStream_t stream) {
    if (!dq) return FA_ERR_NULL;
    fa_status s = check_bwd(kConvert, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, dq, nullptr, nullptr,
                            workspace, workspace_bytes, B, Hq, Hq, N, d, 0, scale);
    if (s != FA_OK) return s;
    fa::BwdParams p = bwd_params(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, dq, nullptr, nullptr,
                                 workspace, B, Hq, Hq, N, 0, scale);
    set_fused_accumulator(p, workspace, B, Hq, N);
    return launched(fa::launch_bwd_dq_convert(p, d, stream));
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
        case FA_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than the required workspace bytes";
        case FA_ERR_ALIAS: return "an output overlaps an input or another output";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_WINDOW: return "window must be >= 0";
        case FA_ERR_SCRATCH:
            return "B * Hq * N exceeds the 2^21 query rows of the no-allocation backward's static scratch";
    }
    return "unknown status";
}

}  // extern "C"
