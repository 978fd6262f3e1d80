// Backward kernels: preprocess (D = rowsum(dO * O)), dK/dV, dQ.
//
// The method recomputes the score and probability tiles from the small per-row
// statistic saved by the forward pass instead of storing the N x N matrices
// (lecture summary, "推导 FlashAttention 的在线 softmax": the backward pass rebuilds
// what it needs from the saved smaller information; code-corey Q38, section
// 2.(2) 重计算: S and softmax are not stored, they are recomputed per tile).
// With the saved natural-log LSE, P_ij = exp(scale * q_i.k_j - LSE_i) exactly,
// and the softmax-Jacobian gradients are (the pages print none; calculus):
//   dP = dO V^T,  D_i = sum_j P_ij dP_ij = dO_i . O_i,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
//
// gfx950 mapping:
//   * dK/dV kernel: a workgroup owns 128 keys of one KV head (32 per wave, K and
//     V held in registers) and streams 64-row tiles of Q and dO of every query
//     head in the group through LDS (natural and transposed copies).  S = Q K^T
//     is formed with the query on the C rows, so P and dS feed the dV and dK
//     contractions straight from registers; the group sum over query heads
//     happens in the accumulators (no atomics, bit-reproducible).
//   * dQ kernel: a workgroup owns 32*QB query rows per wave of one query head
//     (Q, dO, LSE, D in registers) and streams K/V tiles like the forward;
//     S^T = K Q^T keeps each lane on one query, so LSE and D are lane-local.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// ---------------------------------------------------------------------------------
// D_i = sum_t dO_it * O_it (fp32), D/8 lanes per row, 16 bytes per lane.
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void fa_bwd_pre_kernel(const uint16_t* o, const uint16_t* dO,
                                                              float* dsum, long long rows) {
    constexpr int LPR = D / 8;
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long row = gid / LPR;
    const int sub = (int)(gid % LPR);
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = ld_global16(o + row * D + 8 * sub);
        const u32x4 g = ld_global16(dO + row * D + 8 * sub);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc = __builtin_fmaf(bf16_lo(a[w]), bf16_lo(g[w]), acc);
            acc = __builtin_fmaf(bf16_hi(a[w]), bf16_hi(g[w]), acc);
        }
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && sub == 0) dsum[row] = acc;
}

// ---------------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------------
template <int D>
struct DkdvCfg {
    static constexpr int BK = kWaves * 32;  // keys per workgroup
    static constexpr int BQ = 64;           // query rows per streamed tile
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    using T = Tile64<D>;
    static constexpr int QN = 0;
    static constexpr int QT = QN + T::N_ELEMS;
    static constexpr int GN = QT + T::T_ELEMS;   // dO natural
    static constexpr int GT = GN + T::N_ELEMS;   // dO transposed
    static constexpr int VEC = GT + T::T_ELEMS;  // 64 fp32 LSE*log2e, then 64 fp32 D
    static constexpr int STAGE = VEC + 2 * 64 * 2;
};

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkdv_kernel(BwdParams p) {
    using C = DkdvCfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = p.N;
    const int G = p.Hq / p.Hkv;

    const int ntile_k = (N + C::BK - 1) / C::BK;
    int head_kv, kt;
    map_block(blockIdx.x, gridDim.x, ntile_k, p.B * p.Hkv, false, head_kv, kt);
    const int b = head_kv / p.Hkv;
    const int hkv = head_kv % p.Hkv;
    const int k0 = kt * C::BK;
    const int kw0 = k0 + 32 * wave;
    const int key = kw0 + l32;

    const size_t kvoff = (size_t)head_kv * N * D;
    const uint16_t* Kh = (const uint16_t*)p.k + kvoff;
    const uint16_t* Vh = (const uint16_t*)p.v + kvoff;

    // K and V as B operands of S = Q K^T and dP = dO V^T (lane: key, slots: 8 d)
    u32x4 kf[C::DC], vf[C::DC];
#pragma unroll
    for (int c = 0; c < C::DC; ++c) {
        kf[c] = key < N ? ld_global16(Kh + (size_t)key * D + 16 * c + 8 * hh) : zero_u4();
        vf[c] = key < N ? ld_global16(Vh + (size_t)key * D + 16 * c + 8 * hh) : zero_u4();
    }
    f32x16 dkt[C::DB], dvt[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        dkt[db] = zero16();
        dvt[db] = zero16();
    }

    const int nqt = (N + C::BQ - 1) / C::BQ;
    const int qt_start = p.causal ? k0 / C::BQ : 0;
    const int per_head = nqt - qt_start;
    const int nitems = G * per_head;
    const float sl2 = p.scale_log2;

    TileRegs<D> qr, gr;
    float vec_reg = 0.f;
    auto load_item = [&](int item) {
        const int hq = hkv * G + item / per_head;
        const int q0 = (qt_start + item % per_head) * C::BQ;
        const size_t qoff = ((size_t)(b * p.Hq + hq) * N + q0) * D;
        tile_load<D>(qr, (const uint16_t*)p.q + qoff, N - q0, tid);
        tile_load<D>(gr, (const uint16_t*)p.dO + qoff, N - q0, tid);
        const size_t roff = (size_t)(b * p.Hq + hq) * N + q0;
        if (tid < 64) vec_reg = q0 + tid < N ? p.lse[roff + tid] * kLog2e : 0.f;
        else if (tid < 128) vec_reg = q0 + tid - 64 < N ? p.dsum[roff + tid - 64] : 0.f;
    };
    auto store_item = [&](uint16_t* st) {
        tile_store_natural<D>(qr, st + C::QN, tid);
        tile_store_transposed<D>(qr, st + C::QT, tid);
        tile_store_natural<D>(gr, st + C::GN, tid);
        tile_store_transposed<D>(gr, st + C::GT, tid);
        if (tid < 128) ((float*)(st + C::VEC))[tid] = vec_reg;
    };

    if (nitems > 0) {
        load_item(0);
        store_item(smem);
    }
    __syncthreads();

    for (int it = 0; it < nitems; ++it) {
        const bool more = it + 1 < nitems;
        if (more) load_item(it + 1);
        const uint16_t* st = smem + (it & 1) * C::STAGE;
        const int q0 = (qt_start + it % per_head) * C::BQ;

        if (kw0 < N && (!p.causal || q0 + C::BQ - 1 >= kw0)) {
            // ---- S = Q K^T and dP = dO V^T with queries on the C rows
            f32x16 s[2], dp[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                s[qb] = zero16();
                dp[qb] = zero16();
            }
#pragma unroll
            for (int c = 0; c < C::DC; ++c)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    s[qb] = mfma32x32x16(frag_natural<D>(st + C::QN, 32 * qb + l32, c, hh), kf[c], s[qb]);
                    dp[qb] = mfma32x32x16(frag_natural<D>(st + C::GN, 32 * qb + l32, c, hh), vf[c], dp[qb]);
                }

            // ---- P = 2^(S*sl2 - LSE2), dS = P (dP - D)
            const bool need_mask = (p.causal && q0 < kw0 + 31) || (q0 + C::BQ > N);
            const float* lse2 = (const float*)(st + C::VEC);
            const float* dvec = lse2 + 64;
            u32x4 pf[2][2], dsf[2][2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float pv[16], dsv[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 L = *(const f32x4*)(lse2 + 32 * qb + 8 * g + 4 * hh);
                    const f32x4 Dd = *(const f32x4*)(dvec + 32 * qb + 8 * g + 4 * hh);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 4 * g + i;
                        float pr = fast_exp2(__builtin_fmaf(s[qb][r], sl2, -L[i]));
                        if (need_mask) {
                            const int q = q0 + 32 * qb + 8 * g + 4 * hh + i;
                            pr = (q < N && (!p.causal || key <= q)) ? pr : 0.f;
                        }
                        pv[r] = pr;
                        dsv[r] = pr * (dp[qb][r] - Dd[i]);
                    }
                }
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pf[qb][h2][j] = pack_bf16(pv[8 * h2 + 2 * j], pv[8 * h2 + 2 * j + 1]);
                        dsf[qb][h2][j] = pack_bf16(dsv[8 * h2 + 2 * j], dsv[8 * h2 + 2 * j + 1]);
                    }
            }

            // ---- dV^T += dO^T P,  dK^T += Q^T dS   (contractions over the query rows)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const u32x4 ga = frag_transposed<D>(st + C::GT, 32 * db + l32, 32 * qb + 16 * h2, hh);
                        dvt[db] = mfma32x32x16(ga, pf[qb][h2], dvt[db]);
                        const u32x4 qa = frag_transposed<D>(st + C::QT, 32 * db + l32, 32 * qb + 16 * h2, hh);
                        dkt[db] = mfma32x32x16(qa, dsf[qb][h2], dkt[db]);
                    }
        }

        if (more) store_item(smem + ((it + 1) & 1) * C::STAGE);
        __syncthreads();
    }

    if (key < N) {
        uint16_t* dKh = (uint16_t*)p.dk + kvoff + (size_t)key * D;
        uint16_t* dVh = (uint16_t*)p.dv + kvoff + (size_t)key * D;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hh;
                *(u32x2*)(dKh + d0) = u32x2{pack_bf16(dkt[db][4 * g] * sc, dkt[db][4 * g + 1] * sc),
                                            pack_bf16(dkt[db][4 * g + 2] * sc, dkt[db][4 * g + 3] * sc)};
                *(u32x2*)(dVh + d0) = u32x2{pack_bf16(dvt[db][4 * g], dvt[db][4 * g + 1]),
                                            pack_bf16(dvt[db][4 * g + 2], dvt[db][4 * g + 3])};
            }
    }
}

// ---------------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------------
template <int D, int QB>
struct DqCfg {
    static constexpr int BR = kWaves * 32 * QB;
    static constexpr int BC = 64;
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    using T = Tile64<D>;
    static constexpr int KN = 0;
    static constexpr int KT = KN + T::N_ELEMS;
    static constexpr int VN = KT + T::T_ELEMS;
    static constexpr int STAGE = VN + T::N_ELEMS;
};

constexpr int kDqQB = 1;

template <int D, int QB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dq_kernel(BwdParams p) {
    using C = DqCfg<D, QB>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = p.N;

    const int ntile_q = (N + C::BR - 1) / C::BR;
    int head, qt;
    map_block(blockIdx.x, gridDim.x, ntile_q, p.B * p.Hq, p.causal != 0, head, qt);
    const int hq = head % p.Hq;
    const int b = head / p.Hq;
    const int hkv = hq / (p.Hq / p.Hkv);
    const size_t qoff = (size_t)head * N * D;
    const size_t kvoff = ((size_t)b * p.Hkv + hkv) * N * D;
    const uint16_t* Kh = (const uint16_t*)p.k + kvoff;
    const uint16_t* Vh = (const uint16_t*)p.v + kvoff;

    const int q0 = qt * C::BR;
    const int qw0 = q0 + wave * 32 * QB;
    const int q_last = min(q0 + C::BR, N) - 1;
    const int ntiles = p.causal ? q_last / C::BC + 1 : (N + C::BC - 1) / C::BC;
    const int wq_last = min(qw0 + 32 * QB, N) - 1;
    const int wave_tiles = wq_last < qw0 ? 0 : (p.causal ? wq_last / C::BC + 1 : ntiles);

    u32x4 qf[QB][C::DC], gf[QB][C::DC];
    float lse2[QB], dd[QB];
    f32x16 dqt[C::DB][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int q = qw0 + 32 * qb + l32;
        const bool ok = q < N;
#pragma unroll
        for (int c = 0; c < C::DC; ++c) {
            qf[qb][c] = ok ? ld_global16((const uint16_t*)p.q + qoff + (size_t)q * D + 16 * c + 8 * hh) : zero_u4();
            gf[qb][c] = ok ? ld_global16((const uint16_t*)p.dO + qoff + (size_t)q * D + 16 * c + 8 * hh) : zero_u4();
        }
        lse2[qb] = ok ? p.lse[(size_t)head * N + q] * kLog2e : 0.f;
        dd[qb] = ok ? p.dsum[(size_t)head * N + q] : 0.f;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) dqt[db][qb] = zero16();
    }
    const float sl2 = p.scale_log2;

    TileRegs<D> kr, vr;
    tile_load<D>(kr, Kh, N, tid);
    tile_load<D>(vr, Vh, N, tid);
    tile_store_natural<D>(kr, smem + C::KN, tid);
    tile_store_transposed<D>(kr, smem + C::KT, tid);
    tile_store_natural<D>(vr, smem + C::VN, tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * C::BC;
        const bool more = t + 1 < ntiles;
        if (more) {
            tile_load<D>(kr, Kh + (size_t)(k0 + C::BC) * D, N - (k0 + C::BC), tid);
            tile_load<D>(vr, Vh + (size_t)(k0 + C::BC) * D, N - (k0 + C::BC), tid);
        }
        const uint16_t* st = smem + (t & 1) * C::STAGE;

        if (t < wave_tiles) {
            f32x16 s[2][QB], dp[2][QB];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    s[kb][qb] = zero16();
                    dp[kb][qb] = zero16();
                }
#pragma unroll
            for (int c = 0; c < C::DC; ++c)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u32x4 ka = frag_natural<D>(st + C::KN, 32 * kb + l32, c, hh);
                    const u32x4 va = frag_natural<D>(st + C::VN, 32 * kb + l32, c, hh);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        s[kb][qb] = mfma32x32x16(ka, qf[qb][c], s[kb][qb]);
                        dp[kb][qb] = mfma32x32x16(va, gf[qb][c], dp[kb][qb]);
                    }
                }

            const bool need_mask = (p.causal && k0 + C::BC - 1 > qw0) || (k0 + C::BC > N);
            u32x4 dsf[QB][2][2];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int q = qw0 + 32 * qb + l32;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    float dsv[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float pr = fast_exp2(__builtin_fmaf(s[kb][qb][r], sl2, -lse2[qb]));
                        if (need_mask) {
                            const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                            pr = (kk < N && (!p.causal || kk <= q)) ? pr : 0.f;
                        }
                        dsv[r] = pr * (dp[kb][qb][r] - dd[qb]);
                    }
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            dsf[qb][kb][h2][j] = pack_bf16(dsv[8 * h2 + 2 * j], dsv[8 * h2 + 2 * j + 1]);
                }
            }

            // ---- dQ^T += K^T dS^T  (contraction over the keys)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const u32x4 ka = frag_transposed<D>(st + C::KT, 32 * db + l32, 32 * kb + 16 * h2, hh);
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) dqt[db][qb] = mfma32x32x16(ka, dsf[qb][kb][h2], dqt[db][qb]);
                    }
        }

        if (more) {
            uint16_t* nb = smem + ((t + 1) & 1) * C::STAGE;
            tile_store_natural<D>(kr, nb + C::KN, tid);
            tile_store_transposed<D>(kr, nb + C::KT, tid);
            tile_store_natural<D>(vr, nb + C::VN, tid);
        }
        __syncthreads();
    }

    const float sc = p.scale;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int q = qw0 + 32 * qb + l32;
        if (q < N) {
            uint16_t* dQh = (uint16_t*)p.dq + qoff + (size_t)q * D;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *(u32x2*)(dQh + 32 * db + 8 * g + 4 * hh) =
                        u32x2{pack_bf16(dqt[db][qb][4 * g] * sc, dqt[db][qb][4 * g + 1] * sc),
                              pack_bf16(dqt[db][qb][4 * g + 2] * sc, dqt[db][qb][4 * g + 3] * sc)};
        }
    }
}

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------
long long bwd_grid_max(int B, int Hq, int Hkv, int N, int d) {
    const long long pre = ((long long)B * Hq * N * (d / 8) + kThreads - 1) / kThreads;
    const long long dkdv = (long long)B * Hkv * ((N + 127) / 128);
    const long long dq = (long long)B * Hq * ((N + kWaves * 32 * kDqQB - 1) / (kWaves * 32 * kDqQB));
    long long m = pre > dkdv ? pre : dkdv;
    return m > dq ? m : dq;
}

template <int D>
static hipError_t launch_pre(const BwdParams& p, hipStream_t stream) {
    const long long rows = (long long)p.B * p.Hq * p.N;
    const unsigned blocks = (unsigned)((rows * (D / 8) + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(fa_bwd_pre_kernel<D>, dim3(blocks), dim3(kThreads), 0, stream,
                       (const uint16_t*)p.o, (const uint16_t*)p.dO, p.dsum, rows);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv(const BwdParams& p, hipStream_t stream) {
    const unsigned blocks = (unsigned)((long long)p.B * p.Hkv * ((p.N + DkdvCfg<D>::BK - 1) / DkdvCfg<D>::BK));
    hipLaunchKernelGGL(fa_bwd_dkdv_kernel<D>, dim3(blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dq(const BwdParams& p, hipStream_t stream) {
    constexpr int br = DqCfg<D, kDqQB>::BR;
    const unsigned blocks = (unsigned)((long long)p.B * p.Hq * ((p.N + br - 1) / br));
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, kDqQB>), dim3(blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdParams& p, int d, hipStream_t stream) {
    return d == 64 ? launch_pre<64>(p, stream) : launch_pre<128>(p, stream);
}
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, hipStream_t stream) {
    return d == 64 ? launch_dkdv<64>(p, stream) : launch_dkdv<128>(p, stream);
}
hipError_t launch_bwd_dq(const BwdParams& p, int d, hipStream_t stream) {
    return d == 64 ? launch_dq<64>(p, stream) : launch_dq<128>(p, stream);
}

}  // namespace fa
