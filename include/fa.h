/*
 * fa.h: C ABI of libfa_mi355x.so, exact IO-aware attention for MI355X (gfx950).
 *
 * What is computed (the plain definition; the kernels reach it up to rounding):
 *
 *   for every batch b, query head hq and query row i, with g = hq / (Hq / Hkv):
 *     s_ij   = scale * sum_t Q[b,hq,i,t] * K[b,g,j,t]       over visible keys j
 *     visible: all j < N, or j <= i when causal
 *     O[b,hq,i,:] = sum_j softmax_j(s_ij) * V[b,g,j,:]
 *     LSE[b,hq,i] = log(sum_j exp(s_ij))                     (natural log, fp32)
 *
 * Sources (page title, section):
 *   - "ZeRO 与 FlashAttention 各优化什么?" (wushixiongai.com), "注意力瓶颈与优化路线":
 *     FlashAttention / fused SDPA computes exact dense attention with tiling, online
 *     softmax and fusion, cutting HBM traffic and auxiliary storage.
 *   - "LLM interview question bank" ch.029 (ricardokevins.github.io), #36
 *     "FlashAttention 为什么常被说成是 IO-aware", sections 2-3: Q, K, V in
 *     R^(B x H x L x d); Q tiles loop over K/V tiles held on chip with running
 *     (m, l) statistics; the score tile is never written to HBM.
 *   - Stanford lecture summary (youtublog.net): "GPU 显存和注意力瓶颈" (causal: a token
 *     attends to itself and earlier tokens), "推导 FlashAttention 的在线 softmax"
 *     (rescaled numerator/denominator; the backward pass recomputes from a small
 *     saved statistic), "减少缓存表示并验证草稿" (H query heads share G KV heads).
 *
 * Conventions for every entry point:
 *   - Device pointers, contiguous row-major tensors with the head dimension d
 *     fastest: Q, O, dO, dQ are [B, Hq, N, d]; K, V, dK, dV are [B, Hkv, N, d];
 *     LSE is [B, Hq, N] fp32.  Every pointer must be 16-byte aligned.
 *   - Hq must be a multiple of Hkv; query head hq reads KV head hq / (Hq/Hkv)
 *     (contiguous groups).  d must be 64 or 128.  B, Hq, Hkv, N >= 1.
 *   - scale must be finite and >= 0.  causal must be 0 or 1.
 *   - The caller allocates and frees all memory.  The library allocates nothing and
 *     never synchronises: work is enqueued on `stream` (0 = the null stream) and
 *     results are valid after the caller synchronises that stream.  Its only mutable
 *     global state is the static scratch array of fa_backward_noalloc and that array's
 *     per-device address, looked up once under a lock.  Outputs must not overlap
 *     inputs or each other.
 *   - Arguments are validated on the host before anything is launched; on error
 *     nothing is launched and no output is touched.  FA_ERR_LAUNCH reports a
 *     launch failure seen by hipGetLastError; faults inside a kernel surface at
 *     the caller's next synchronisation, as usual for HIP.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,       /* a required pointer is NULL                        */
    FA_ERR_SHAPE = 2,      /* B, Hq, Hkv or N < 1, or the launch grid too large  */
    FA_ERR_GQA = 3,        /* Hq is not a multiple of Hkv                        */
    FA_ERR_HEADDIM = 4,    /* d is not 64 or 128                                 */
    FA_ERR_SCALE = 5,      /* scale is NaN, infinite or negative                 */
    FA_ERR_ALIGN = 6,      /* a pointer is not 16-byte aligned                   */
    FA_ERR_FLAG = 7,       /* causal is not 0 or 1                               */
    FA_ERR_WORKSPACE = 8,  /* workspace NULL, misaligned or too small            */
    FA_ERR_ALIAS = 9,      /* an output overlaps an input or another output     */
    FA_ERR_LAUNCH = 10,    /* hipGetLastError reported a launch failure          */
    FA_ERR_WINDOW = 11,    /* window is negative                                 */
    FA_ERR_SCRATCH = 12    /* larger than the no-allocation entry point's scratch */
} fa_status;

/*
 * Forward pass, bf16 inputs and outputs, fp32 accumulation and softmax state.
 * Defined by: "LLM interview question bank" ch.029 #36, sections 2-3 (Q, K, V in
 * R^(B x H x L x d); query tiles walk the K/V tiles with a running max and
 * denominator, the score tile stays on chip, O is written once); lecture summary,
 * "GPU 显存和注意力瓶颈" (the causal rule, diagonal included) and "减少缓存表示并验证草稿"
 * (Hq query heads over Hkv key/value heads); "推导 FlashAttention 的在线 softmax" (the
 * small per-row statistic kept for the backward pass: here the natural-log LSE).
 * q [B,Hq,N,d], k and v [B,Hkv,N,d] (bf16, read only); o [B,Hq,N,d] bf16 and
 * lse [B,Hq,N] fp32 are overwritten.  P is rounded to bf16 (round to nearest
 * even) before the P.V contraction, and O is rounded to bf16 on store.
 * Errors: FA_ERR_NULL, _SHAPE, _GQA, _HEADDIM, _FLAG, _SCALE, _ALIGN, _ALIAS
 * (nothing launched), FA_ERR_LAUNCH.
 */
fa_status fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                     hipStream_t stream);

/*
 * Forward pass with every tensor and every intermediate in fp32 (no reduced
 * precision anywhere).  Same definition and sources as fa_forward (the pages fix no
 * precision; this is the path held to 1e-5 of the exact result).  Same shapes, layout,
 * rules and errors as fa_forward, with 4-byte elements.
 */
fa_status fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                         int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                         hipStream_t stream);

/*
 * Validation diagnostic (not a production path): exactly fa_forward's kernel and
 * arithmetic, but O is stored as fp32 [B,Hq,N,d] (the value fa_forward rounds to
 * bf16), so a test can separate the kernel's own error from the bf16 rounding of the
 * stored output: rounding this O to bf16 (nearest even) gives fa_forward's O bit for
 * bit.  q, k, v bf16 as for fa_forward; lse as for fa_forward.  Same rules and errors.
 */
fa_status fa_forward_fp32_out(const void* q, const void* k, const void* v, float* o, float* lse,
                              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                              hipStream_t stream);

/* Bytes of device workspace fa_backward needs: two fp32 per query row r of
 * R = B*Hq*N (the per-row term D_r = sum_t dO_rt * O_rt, then LSE_r in base-2 units;
 * lecture summary, "推导 FlashAttention 的在线 softmax": the backward pass rebuilds P
 * from the small saved statistic), 8*R bytes.  Returns 0 for invalid sizes (B, Hq or
 * N < 1). */
size_t fa_backward_workspace_bytes(int B, int Hq, int N);

/*
 * Backward pass for L with upstream gradient dO = dL/dO, bf16, recomputing P
 * tile by tile from the saved lse (the small statistic the forward keeps).
 * Defined by: code-corey Q38, section 2.(2) 重计算 (S and P are not stored, they are
 * recomputed in the backward pass); lecture summary, "推导 FlashAttention 的在线
 * softmax" (the backward pass works from the saved statistic); "LLM interview question
 * bank" ch.029 #36, section 7 (the backward costs 2.2-2.5x the forward).  The
 * gradients are the softmax-Jacobian ones (the pages print none):
 *   dP = dO V^T,  D_i = sum_j P_ij dP_ij = dO_i . O_i,  dS = P * (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
 * q, k, v, o, dO (bf16) and lse (fp32) are the forward's inputs and outputs.
 * dq [B,Hq,N,d] and dk, dv [B,Hkv,N,d] (bf16) are overwritten (not accumulated);
 * dk and dv of a KV head are the sums over the Hq/Hkv query heads of its group.
 * workspace: device memory of at least fa_backward_workspace_bytes(B,Hq,N)
 * bytes (passed in workspace_bytes), 16-byte aligned, clobbered by the call.
 * It enqueues fa_backward_preprocess_dq, then fa_backward_dkdv; the results are
 * bit-identical to fa_backward_preprocess + fa_backward_dkdv + fa_backward_dq, and
 * every output is bit-reproducible from run to run.
 * Errors: those of fa_forward, and FA_ERR_WORKSPACE (NULL, misaligned or smaller
 * than required); the workspace may overlap no tensor argument (FA_ERR_ALIAS).
 */
fa_status fa_backward(const void* q, const void* k, const void* v, const void* o,
                      const void* dO, const float* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes,
                      int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                      hipStream_t stream);

/*
 * Alternative backward with the same definition, arguments and results as fa_backward
 * (code-corey Q38, section 2.(2) 重计算: recompute instead of store; here S and dP are
 * formed once per (query, key) pair for all three gradients).  One kernel forms dK,
 * dV and dQ: each query row's dQ contribution of a key block is added in fp32 with
 * atomic adds to an accumulator in the workspace, which a last kernel scales into bf16
 * dq.  Five contractions per pair instead of fa_backward's seven, but on MI355X the
 * fp32 atomic traffic (4 bytes per query row, d and key block of 128) makes it slower
 * than fa_backward at the sizes measured; dk and dv are bit-reproducible, dq may differ
 * in its last bits from run to run (the order of the fp32 adds is not fixed).
 * workspace: at least fa_backward_fused_workspace_bytes(B,Hq,N,d) bytes: the
 * per-row terms of fa_backward, then from the next 256-byte boundary the fp32 dQ
 * accumulator [B*Hq*N][d].  Enqueues fa_backward_preprocess, fa_backward_dkdv_dq and
 * fa_backward_dq_convert.  Other rules and errors as for fa_backward.
 */
size_t fa_backward_fused_workspace_bytes(int B, int Hq, int N, int d);
fa_status fa_backward_fused(const void* q, const void* k, const void* v, const void* o,
                            const void* dO, const float* lse, void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes,
                            int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                            hipStream_t stream);

/*
 * fa_backward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument and no allocation of any kind.  The per-row terms (D and LSE in base 2,
 * 8 bytes per query row) go to a static device array of the library, 2^21 query rows
 * (16 MiB) on every device the library runs on, held until the process ends; calls with
 * B*Hq*N above 2^21 return FA_ERR_SCRATCH and launch nothing.  The array's address on
 * the stream's device is looked up on the first call on that device.  Every call on a
 * device shares that device's array: two calls that overlap in time on one device
 * (e.g. on two streams) race and give wrong gradients; calls on one stream, or
 * otherwise ordered, are safe (each call overwrites every row it reads).  Results are
 * bit-identical to fa_backward_preprocess + fa_backward_dkdv + fa_backward_dq.  Other
 * arguments, rules and errors as for fa_backward.
 */
fa_status fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                              hipStream_t stream);

/*
 * The backward's steps (same sources as fa_backward: the preprocess forms the per-row
 * term of the softmax Jacobian, D_i = dO_i . O_i; the others recompute P from the saved
 * statistic), exposed so that a caller can place and time them itself.  Arguments,
 * layouts and errors are those of fa_backward.
 *   fa_backward_preprocess: for every query row (b, h, i), row index
 *     r = (b*Hq + h)*N + i, workspace as fp32 [2][B*Hq*N] at its start:
 *     workspace[r] = D_r = sum_t dO_r,t * O_r,t and
 *     workspace[B*Hq*N + r] = lse[r] * log2(e); when workspace_bytes is at least
 *     fa_backward_fused_workspace_bytes(B,Hq,N,d), it also zeroes the fused
 *     alternative's dQ accumulator.
 *   fa_backward_dkdv: dk, dv from q, k, v, dO and the preprocessed workspace;
 *   fa_backward_dq:   dq from q, k, v, dO and the preprocessed workspace
 *     (these two only read the workspace and may run concurrently on two streams);
 *   fa_backward_preprocess_dq: fa_backward_preprocess and fa_backward_dq in one
 *     kernel: each dQ workgroup forms the per-row terms of its own rows (from o, dO and
 *     lse, bit for bit as fa_backward_preprocess does, without the fused alternative's
 *     accumulator), writes them to the workspace and uses them; fa_backward_dkdv may
 *     follow once it has completed.  This is the order fa_backward takes.
 *   fa_backward_dkdv_dq (fused alternative, workspace of
 *     fa_backward_fused_workspace_bytes): dk, dv, and every row's dQ contribution added
 *     (unscaled, fp32) into the accumulator, which it requires zeroed by the preprocess;
 *   fa_backward_dq_convert: dq = scale * accumulator, rounded to bf16.
 * The kernels after the preprocess read the saved statistic only through the
 * workspace, so it must come from fa_backward_preprocess (or
 * fa_backward_preprocess_dq) of the same o, dO and lse.
 */
fa_status fa_backward_preprocess(const void* o, const void* dO, const float* lse, void* workspace,
                                 size_t workspace_bytes, int B, int Hq, int N, int d, hipStream_t stream);
fa_status fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dO,
                           const void* workspace, size_t workspace_bytes,
                           void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int causal,
                           float scale, hipStream_t stream);
fa_status fa_backward_dq(const void* q, const void* k, const void* v, const void* dO,
                         const void* workspace, size_t workspace_bytes,
                         void* dq, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                         hipStream_t stream);
fa_status fa_backward_preprocess_dq(const void* q, const void* k, const void* v, const void* o,
                                    const void* dO, const float* lse, void* workspace,
                                    size_t workspace_bytes, void* dq, int B, int Hq, int Hkv, int N,
                                    int d, int causal, float scale, hipStream_t stream);
fa_status fa_backward_dkdv_dq(const void* q, const void* k, const void* v, const void* dO,
                              void* workspace, size_t workspace_bytes, void* dk, void* dv,
                              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                              hipStream_t stream);
fa_status fa_backward_dq_convert(const void* workspace, size_t workspace_bytes, void* dq,
                                 int B, int Hq, int N, int d, float scale, hipStream_t stream);

/*
 * Sliding-window attention: as fa_forward / fa_backward (and its dK/dV and dQ
 * steps), with key j visible to query i only if |i - j| <= window, on top of the
 * causal rule; a causal row thus sees its window + 1 most recent keys (page "ZeRO 与
 * FlashAttention 各优化什么?", "注意力瓶颈与优化路线": a sliding window limits the
 * positions a query sees and the work done).  window >= 0 (FA_ERR_WINDOW otherwise);
 * a window of N - 1 or more is no restriction.  Tiles wholly outside the band are
 * neither loaded nor computed.  Other arguments, layouts and errors are those of the
 * calls without a window; the backward takes lse from fa_forward_window with the same
 * window, the dK/dV and dQ steps take the workspace of fa_backward_preprocess, and
 * fa_backward_preprocess_dq_window is fa_backward_preprocess_dq with the window.
 */
fa_status fa_forward_window(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                            hipStream_t stream);
fa_status fa_backward_window(const void* q, const void* k, const void* v, const void* o,
                             const void* dO, const float* lse, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes,
                             int B, int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                             hipStream_t stream);
fa_status fa_backward_dkdv_window(const void* q, const void* k, const void* v, const void* dO,
                                  const void* workspace, size_t workspace_bytes,
                                  void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int causal,
                                  int window, float scale, hipStream_t stream);
fa_status fa_backward_dq_window(const void* q, const void* k, const void* v, const void* dO,
                                const void* workspace, size_t workspace_bytes,
                                void* dq, int B, int Hq, int Hkv, int N, int d, int causal,
                                int window, float scale, hipStream_t stream);
fa_status fa_backward_preprocess_dq_window(const void* q, const void* k, const void* v,
                                           const void* o, const void* dO, const float* lse,
                                           void* workspace, size_t workspace_bytes, void* dq,
                                           int B, int Hq, int Hkv, int N, int d, int causal,
                                           int window, float scale, hipStream_t stream);


/*
 * Block-sparse attention: as fa_forward / fa_backward (and its dK/dV and dQ steps),
 * with key j visible to query i only if block_mask[(i/64)*nb + j/64] is nonzero, on
 * top of the causal rule (page "ZeRO 与 FlashAttention 各优化什么?",
 * "注意力瓶颈与优化路线": block-sparse and global + local patterns compute only part of
 * the positions).  block_mask: device bytes [nb][nb], nb = ceil(N/64) <= 2048 (so
 * N <= 131072, FA_ERR_SHAPE beyond), shared by every batch and head, read only.
 * Blocks whose byte is 0 are neither loaded nor computed.  A query that sees no key
 * gets O = 0 and LSE = -inf, and contributes nothing to the gradients.  Other
 * arguments, layouts and errors are those of the dense calls; the backward takes lse
 * from fa_forward_blocksparse with the same layout, the dK/dV and dQ steps take
 * the workspace of fa_backward_preprocess, and fa_backward_preprocess_dq_blocksparse
 * is fa_backward_preprocess_dq with the layout.  fa_backward_blocksparse enqueues
 * fa_backward_preprocess, then the dK/dV and dQ steps (same results as the order
 * fa_backward takes, bit for bit).
 */
fa_status fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const unsigned char* block_mask,
                                 int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                                 hipStream_t stream);
fa_status fa_backward_blocksparse(const void* q, const void* k, const void* v, const void* o,
                                  const void* dO, const float* lse, void* dq, void* dk, void* dv,
                                  const unsigned char* block_mask, void* workspace, size_t workspace_bytes,
                                  int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                                  hipStream_t stream);
fa_status fa_backward_dkdv_blocksparse(const void* q, const void* k, const void* v, const void* dO,
                                       const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                                       const unsigned char* block_mask,
                                       int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                                       hipStream_t stream);
fa_status fa_backward_dq_blocksparse(const void* q, const void* k, const void* v, const void* dO,
                                     const void* workspace, size_t workspace_bytes, void* dq,
                                     const unsigned char* block_mask,
                                     int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                                     hipStream_t stream);
fa_status fa_backward_preprocess_dq_blocksparse(const void* q, const void* k, const void* v,
                                                const void* o, const void* dO, const float* lse,
                                                void* workspace, size_t workspace_bytes, void* dq,
                                                const unsigned char* block_mask,
                                                int B, int Hq, int Hkv, int N, int d, int causal,
                                                float scale, hipStream_t stream);

/*
 * Decode forward: Nq new queries per head against a cache of Nk keys and values.
 *
 * The queries are the last Nq tokens of a sequence whose Nk keys and values, their
 * own included, are all in the cache (Stanford lecture summary, "衡量并优化推理":
 * decoding reuses the keys and values of earlier tokens).  Query i sits at
 * position Nk - Nq + i; when causal it sees keys j <= Nk - Nq + i, otherwise all
 * Nk keys.  With Nq = Nk this is exactly fa_forward.  Per query row:
 *     O[b,hq,i,:] = sum_j softmax_j(s_ij) V[b,g,j,:],  LSE[b,hq,i] = log sum_j exp(s_ij)
 * with s_ij and g as above.
 *   q [B,Hq,Nq,d] bf16, k and v [B,Hkv,Nk,d] bf16 (read only); o [B,Hq,Nq,d] bf16
 *   and lse [B,Hq,Nq] fp32 are overwritten.  Nq >= 1, Nk >= 1, and Nq <= Nk
 *   when causal (FA_ERR_SHAPE otherwise); other rules as for fa_forward.
 *   workspace: device memory of at least fa_decode_workspace_bytes(...) bytes
 *   (passed in workspace_bytes), 16-byte aligned, clobbered by the call; it holds
 *   the partial results of the key ranges the cache is cut into, which a second
 *   kernel merges by their log-sum-exp.
 * Bound by HBM bandwidth: every K and V byte is read once per call, shared by
 * the Hq/Hkv query heads of its group.
 */
fa_status fa_decode_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                            void* workspace, size_t workspace_bytes,
                            int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                            hipStream_t stream);

/* Bytes of device workspace fa_decode_forward (and fa_decode_paged_forward, with Nk
 * its max_seq_len) needs for these sizes (it depends on the sizes only); 0 for
 * invalid sizes. */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/*
 * The two kernels fa_decode_forward enqueues, in this order, exposed so that a
 * caller can time or place each one: fa_decode_split computes every key range's
 * partial result into the workspace, fa_decode_merge combines them into o and lse.
 * Both take fa_decode_forward's arguments and rules, and the merge must follow a
 * split with the same arguments and workspace.  When the sizes give a single key
 * range, the split writes o and lse itself and the merge enqueues nothing.
 */
fa_status fa_decode_split(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                          hipStream_t stream);
fa_status fa_decode_merge(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                          hipStream_t stream);

/*
 * Decode forward against a paged key/value cache (Stanford lecture summary,
 * "衡量并优化推理": the cache is cut into fixed-size blocks and metadata maps a
 * sequence's logical token positions to physical blocks, so that memory is taken per
 * block rather than reserved for the longest possible sequence).
 *   k_pages, v_pages: bf16 pools [num_pages, Hkv, page_size, d]; page p holds
 *     page_size consecutive tokens of every KV head.
 *   block_table: int32 [B, max_blocks] (device); token t of sequence b is row
 *     t % page_size of page block_table[b*max_blocks + t/page_size].
 *   seq_lens: int32 [B] (device); sequence b has seq_lens[b] cached tokens, its Nq
 *     queries sit at positions seq_lens[b] - Nq + i (as in fa_decode_forward).
 *   max_seq_len: an upper bound of every seq_lens[b], known on the host: the key
 *     splits and the workspace (fa_decode_workspace_bytes(B, Hq, Hkv, Nq,
 *     max_seq_len, d)) are sized from it; larger lengths are cut to it.
 *   q, o [B,Hq,Nq,d] bf16; lse [B,Hq,Nq] fp32.  page_size must be a multiple of
 *   64 and max_blocks*page_size >= max_seq_len (FA_ERR_SHAPE otherwise);
 *   block_table and seq_lens need 4-byte alignment, the rest 16 bytes.
 * Tables are read on the device: a table entry outside [0, num_pages) contributes
 * no keys (it is never dereferenced), and a query with no visible key (a sequence
 * shorter than its queries under the causal rule) gets O = 0 and LSE = -inf.
 * fa_decode_paged_split / _merge are its two kernels, as for fa_decode_forward.
 */
fa_status fa_decode_paged_forward(const void* q, const void* k_pages, const void* v_pages,
                                  const int* block_table, const int* seq_lens, void* o, float* lse,
                                  void* workspace, size_t workspace_bytes,
                                  int B, int Hq, int Hkv, int Nq, int max_seq_len, int num_pages,
                                  int page_size, int max_blocks, int d, int causal, float scale,
                                  hipStream_t stream);
fa_status fa_decode_paged_split(const void* q, const void* k_pages, const void* v_pages,
                                const int* block_table, const int* seq_lens, void* o, float* lse,
                                void* workspace, size_t workspace_bytes,
                                int B, int Hq, int Hkv, int Nq, int max_seq_len, int num_pages,
                                int page_size, int max_blocks, int d, int causal, float scale,
                                hipStream_t stream);
fa_status fa_decode_paged_merge(const void* q, const void* k_pages, const void* v_pages,
                                const int* block_table, const int* seq_lens, void* o, float* lse,
                                void* workspace, size_t workspace_bytes,
                                int B, int Hq, int Hkv, int Nq, int max_seq_len, int num_pages,
                                int page_size, int max_blocks, int d, int causal, float scale,
                                hipStream_t stream);

/*
 * Host-only validation of a forward call, exactly as fa_forward performs it
 * (pointer presence, alignment and overlap, shapes, flag, scale), for an
 * element size elt_bytes of 2 (bf16) or 4 (fp32).  Touches no device memory
 * and launches nothing; usable without a GPU.
 */
fa_status fa_check_args(const void* q, const void* k, const void* v, const void* o,
                        const void* lse, int B, int Hq, int Hkv, int N, int d, int causal,
                        float scale, int elt_bytes);

/* Static, human-readable description of a status code. */
const char* fa_status_string(fa_status status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
