// Private interface between the C ABI (fa_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Block-sparse layouts: side of a block and the largest layout (host-side copies of
// the device constants).
constexpr int kSparseBlockHost = 64;
constexpr int kSparseMaxBlocksHost = 2048;

// Workgroup tiles the launch plans are made of (the kernels assert they match).
constexpr int kFwdRows = 256;     // query rows per forward workgroup (8 waves x 32)
constexpr int kFwdF32Rows = 32;   // query rows per fp32 forward workgroup
constexpr int kDkdvKeys = 128;    // keys per dK/dV workgroup
constexpr int kDqRows = 256;      // query rows per dQ workgroup
constexpr int kDecodeTile = 64;   // keys per decode K/V tile
// Decode: one single-wave workgroup per SIMD, four per CU on 256 CUs.  Paged calls plan
// for their longest sequence (the only length the host knows), so with mixed lengths the
// splits past a shorter sequence's end exit at once; planning more, shorter splits
// (2048 to 4096), issuing splits before sequences, or balancing the splits over the
// tokens the sequences hold (lengths read on the device, every SIMD streaming) measured
// slower: the paged split is capped by the memory system's rate for scattered pages.
constexpr int kDecodeTargetWgs = 1024;

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, N, causal;
    int window;         // sliding window: key j visible to query i only if |i - j| <= window; < 0: none
    const uint8_t* block_mask;   // block-sparse layout [nb][nb] over 64 x 64 blocks, or null
    float scale;        // softmax scale
    float scale_log2;   // scale * log2(e)
    float* o32;         // validation only: when set, the dense kernels store O in fp32 here
                        // (the value they would round to bf16) instead of writing o
};

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dO;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* dsum;        // workspace: D_i = dO_i . O_i, one fp32 per query row
    float* lse2;        // workspace: LSE_i * log2(e), one fp32 per query row
    float* dqacc;       // workspace: fp32 dQ accumulator [B*Hq*N][d] of the fused backward
                        // (zeroed by the preprocess when set), or null
    int B, Hq, Hkv, N, causal;
    int window;         // as in FwdParams
    const uint8_t* block_mask;   // as in FwdParams
    float scale;
    float scale_log2;
    int form_rows;      // dQ kernel: form the per-row terms (dsum, lse2) from o, dO and lse
                        // and write them, instead of reading the preprocess's
};

// Decode: Nq queries per head against Nk cached keys, the key range cut into
// `nsplit` splits of `tiles_per_split` 64-key tiles, each split's result merged by
// its log-sum-exp.
struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    float* part_o;      // workspace: fp32 [nsplit][B*Hq*Nq][d], each split's normalised O
    float* part_lse;    // workspace: fp32 [nsplit][B*Hq*Nq], each split's LSE in base 2
    int B, Hq, Hkv, Nq, Nk, causal;   // paged: Nk is the longest sequence the plan covers
    // paged cache (k, v are pools [num_pages][Hkv][page_size][d]): sequence b's token t
    // is row t % page_size of page block_table[b * max_blocks + t / page_size]
    const int* block_table;
    const int* seq_lens;  // [B] tokens of each sequence
    int max_blocks, page_size, num_pages;
    int nrb;            // 32-row blocks of the G*Nq packed query rows of a KV head
    int nsplit, tiles_per_split;
    float scale_log2;
};

struct DecodePlan {
    int nrb, nsplit, tiles_per_split;
    long long grid;           // workgroups of the split kernel
    size_t workspace_bytes;
};
DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d);

long long fwd_bf16_grid(int B, int Hq, int N, int d);
long long fwd_f32_grid(int B, int Hq, int N);
long long bwd_grid_max(int B, int Hq, int Hkv, int N, int d);

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t stream);
enum DecodeSteps { kDecodeSplit = 1, kDecodeMerge = 2 };
hipError_t launch_decode(const DecodeParams& p, int d, int steps, bool paged, hipStream_t stream);
// No-allocation backward: the per-row workspace (D and LSE in base 2) lives in a static
// device array of kScratchRows rows per device.  bwd_scratch returns that array's address
// on the device `stream` belongs to (looked up once per device).
constexpr long long kScratchRows = 1LL << 21;
hipError_t bwd_scratch(hipStream_t stream, float** ptr);
hipError_t launch_bwd_pre(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_fused(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_dq_convert(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_dq_rows(const BwdParams& p, int d, hipStream_t stream);   // dQ forming the per-row terms

}  // namespace fa
