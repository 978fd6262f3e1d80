// Host-side launch plans: grid sizes and workspace sizes for given shapes.  Pure
// arithmetic, no HIP calls, so the argument checks of the C ABI that depend on them
// can also be built and tested on a host without a GPU.
#include <stddef.h>

#include "fa_launch.hpp"

namespace fa {

long long fwd_bf16_grid(int B, int Hq, int N, int /*d*/) {
    return (long long)B * Hq * ((N + kFwdRows - 1) / kFwdRows);
}

long long fwd_f32_grid(int B, int Hq, int N) { return (long long)B * Hq * ((N + kFwdF32Rows - 1) / kFwdF32Rows); }

// The largest grid among the backward kernels: the preprocess (d/8 lanes per query row,
// 256 threads per workgroup), dK/dV (one workgroup per key tile of a KV head) and dQ
// (one per row tile of a query head).
long long bwd_grid_max(int B, int Hq, int Hkv, int N, int d) {
    const long long pre = ((long long)B * Hq * N * (d / 8) + 255) / 256;
    const long long dkdv = (long long)B * Hkv * ((N + kDkdvKeys - 1) / kDkdvKeys);
    const long long dq = (long long)B * Hq * ((N + kDqRows - 1) / kDqRows);
    long long m = pre > dkdv ? pre : dkdv;
    return m > dq ? m : dq;
}

// Decode: the cache of a (batch, KV head) pair is cut into splits of whole 64-key
// tiles so that about kDecodeTargetWgs single-wave workgroups run; each split writes
// its partial O (fp32, d values) and its base-2 LSE for every query row.
DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    DecodePlan pl{};
    const long long target = kDecodeTargetWgs;
    const long long G = Hq / Hkv;
    const long long ntiles = (Nk + kDecodeTile - 1) / kDecodeTile;
    pl.nrb = (int)((G * Nq + 31) / 32);
    const long long units = (long long)B * Hkv * pl.nrb;   // workgroups per split
    long long per = (ntiles * units + target - 1) / target;
    per = per < 1 ? 1 : (per > ntiles ? ntiles : per);
    pl.tiles_per_split = (int)per;
    pl.nsplit = (int)((ntiles + per - 1) / per);
    pl.grid = units * pl.nsplit;
    pl.workspace_bytes = (size_t)pl.nsplit * B * Hq * Nq * (size_t)(d + 1) * sizeof(float);
    return pl;
}

}  // namespace fa
