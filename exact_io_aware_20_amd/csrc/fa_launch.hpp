// Private interface between the C ABI (fa_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, N, causal;
    float scale;        // softmax scale
    float scale_log2;   // scale * log2(e)
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
    int B, Hq, Hkv, N, causal;
    float scale;
    float scale_log2;
};

long long fwd_bf16_grid(int B, int Hq, int N, int d);
long long fwd_f32_grid(int B, int Hq, int N);
long long bwd_grid_max(int B, int Hq, int Hkv, int N, int d);

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_pre(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, int d, hipStream_t stream);

}  // namespace fa
