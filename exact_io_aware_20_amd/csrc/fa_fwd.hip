// Forward kernels: bf16 matrix-core kernel and an all-fp32 kernel.
//
// The method (page "LLM interview question bank" ch.029 #36, section 3, and the
// lecture summary's "推导 FlashAttention 的在线 softmax"): each workgroup owns a tile of
// query rows, walks the key/value tiles in order, keeps the score tile on chip,
// updates a running row maximum m and denominator l, rescales the output
// accumulator by exp(m_old - m_new) when m grows, and writes O once at the end
// together with the per-row log-sum-exp that the backward pass recomputes from.
// Causal tiles that lie entirely above the diagonal are never loaded (lecture
// summary, "GPU 显存和注意力瓶颈": a token sees itself and earlier tokens).
//
// gfx950 mapping of the bf16 kernel:
//   * 4 waves per workgroup, each wave owns 32*QB query rows; K/V tiles of 64
//     keys are staged through LDS (double-buffered, one barrier per tile).
//   * Scores are formed transposed, S^T = K Q^T, so a lane holds one query (its
//     column) and 16 keys; the row maximum is an in-lane max plus one exchange
//     with lane l^32, and the running statistics are lane-local scalars.
//   * O^T = V^T P^T reuses the S^T registers, rounded to bf16, directly as the
//     B operand; V is staged transposed in LDS for the A operand.
//   * Scores are kept in base-2 units (scale*log2 e folded into one FMA before
//     v_exp_f32).  The reference maximum is only moved when a row's maximum
//     grows by more than 2^8 (kRescaleLog2): the quotient O = sum p v / sum p is
//     the same for any reference, p stays <= 256, and the O rescale, which costs
//     d/64 multiplies per score, is skipped on almost every tile.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr float kRescaleLog2 = 8.0f;

template <int D, int QB>
struct FwdCfg {
    static constexpr int BR = kWaves * 32 * QB;   // query rows per workgroup
    static constexpr int BC = 64;                 // keys per K/V tile
    static constexpr int DC = D / 16;             // k-chunks of the S contraction
    static constexpr int DB = D / 32;             // 32-row blocks of O^T
    using T = Tile64<D>;
    static constexpr int K_OFF = 0;
    static constexpr int V_OFF = T::N_ELEMS;
    static constexpr int STAGE = T::N_ELEMS + T::T_ELEMS;
};

template <int D, int QB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_fwd_bf16_kernel(FwdParams p) {
    using C = FwdCfg<D, QB>;
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

    const uint16_t* Qh = (const uint16_t*)p.q + (size_t)head * N * D;
    const uint16_t* Kh = (const uint16_t*)p.k + ((size_t)b * p.Hkv + hkv) * N * D;
    const uint16_t* Vh = (const uint16_t*)p.v + ((size_t)b * p.Hkv + hkv) * N * D;

    const int q0 = qt * C::BR;
    const int qw0 = q0 + wave * 32 * QB;
    const int q_last = min(q0 + C::BR, N) - 1;
    const int ntiles = p.causal ? q_last / C::BC + 1 : (N + C::BC - 1) / C::BC;
    const int wq_last = min(qw0 + 32 * QB, N) - 1;
    const int wave_tiles = wq_last < qw0 ? 0 : (p.causal ? wq_last / C::BC + 1 : ntiles);

    // Q fragments: B operand of S^T = K Q^T (lane: query, slots: 8 consecutive d).
    u32x4 qf[QB][C::DC];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int q = qw0 + 32 * qb + l32;
#pragma unroll
        for (int c = 0; c < C::DC; ++c)
            qf[qb][c] = q < N ? ld_global16(Qh + (size_t)q * D + 16 * c + 8 * hh) : zero_u4();
    }

    f32x16 o[C::DB][QB];
    float m_ref[QB], l_part[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_ref[qb] = kNegInf;
        l_part[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db][qb] = zero16();
    }
    const float sl2 = p.scale_log2;

    TileRegs<D> kr, vr;
    tile_load<D>(kr, Kh, N, tid);
    tile_load<D>(vr, Vh, N, tid);
    tile_store_natural<D>(kr, smem + C::K_OFF, tid);
    tile_store_transposed<D>(vr, smem + C::V_OFF, tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * C::BC;
        const bool more = t + 1 < ntiles;
        if (more) {
            tile_load<D>(kr, Kh + (size_t)(k0 + C::BC) * D, N - (k0 + C::BC), tid);
            tile_load<D>(vr, Vh + (size_t)(k0 + C::BC) * D, N - (k0 + C::BC), tid);
        }
        const uint16_t* Ks = smem + (t & 1) * C::STAGE + C::K_OFF;
        const uint16_t* Vt = smem + (t & 1) * C::STAGE + C::V_OFF;

        if (t < wave_tiles) {
            // ---- S^T = K Q^T : [2 key blocks][QB query blocks] of 32 x 32
            f32x16 s[2][QB];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[kb][qb] = zero16();
#pragma unroll
            for (int c = 0; c < C::DC; ++c) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u32x4 kf = frag_natural<D>(Ks, 32 * kb + l32, c, hh);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32x32x16(kf, qf[qb][c], s[kb][qb]);
                }
            }

            // ---- mask: the causal diagonal and keys past N (ragged last tile)
            const bool need_mask = (p.causal && k0 + C::BC - 1 > qw0) || (k0 + C::BC > N);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int q = qw0 + 32 * qb + l32;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                            const bool vis = key < N && (!p.causal || key <= q);
                            s[kb][qb][r] = vis ? s[kb][qb][r] : kNegInf;
                        }
                }
            }

            // ---- online softmax: row max (in-lane + partner lane), lazy rescale
            float mt[QB];
            bool need = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = kNegInf;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                mt[qb] = mx == kNegInf ? kNegInf : mx * sl2;
                need |= mt[qb] > m_ref[qb] + kRescaleLog2;
            }
            if (__ballot(need)) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const float mnew = mt[qb] > m_ref[qb] + kRescaleLog2 ? mt[qb] : m_ref[qb];
                    const float alpha = m_ref[qb] == kNegInf ? 0.f : fast_exp2(m_ref[qb] - mnew);
                    m_ref[qb] = mnew;
                    l_part[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
                }
            }

            // ---- P = 2^(S*sl2 - m), packed to bf16 as the B operand of O^T = V^T P^T
            u32x4 pf[QB][2][2];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mref = m_ref[qb] == kNegInf ? 0.f : m_ref[qb];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float sa = s[kb][qb][8 * h2 + 2 * j];
                            const float sb = s[kb][qb][8 * h2 + 2 * j + 1];
                            float pa = fast_exp2(__builtin_fmaf(sa, sl2, -mref));
                            float pb = fast_exp2(__builtin_fmaf(sb, sl2, -mref));
                            if (need_mask) {
                                pa = sa == kNegInf ? 0.f : pa;
                                pb = sb == kNegInf ? 0.f : pb;
                            }
                            const uint32_t pk = pack_bf16(pa, pb);
                            pf[qb][kb][h2][j] = pk;
                            l_part[qb] = add_bf16_pair(pk, l_part[qb]);
                        }
            }

            // ---- O^T += V^T P^T
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const u32x4 vf = frag_transposed<D>(Vt, 32 * db + l32, 32 * kb + 16 * h2, hh);
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma32x32x16(vf, pf[qb][kb][h2], o[db][qb]);
                    }
        }

        if (more) {
            uint16_t* nb = smem + ((t + 1) & 1) * C::STAGE;
            tile_store_natural<D>(kr, nb + C::K_OFF, tid);
            tile_store_transposed<D>(vr, nb + C::V_OFF, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l (bf16, round to nearest even), LSE in natural log
    uint16_t* Oh = (uint16_t*)p.o + (size_t)head * N * D;
    float* lse = p.lse + (size_t)head * N;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = l_part[qb] + __shfl_xor(l_part[qb], 32);
        const int q = qw0 + 32 * qb + l32;
        if (q < N) {
            const float inv = 1.0f / lt;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x2 v2 = {pack_bf16(o[db][qb][4 * g] * inv, o[db][qb][4 * g + 1] * inv),
                                      pack_bf16(o[db][qb][4 * g + 2] * inv, o[db][qb][4 * g + 3] * inv)};
                    *(u32x2*)(Oh + (size_t)q * D + 32 * db + 8 * g + 4 * hh) = v2;
                }
            if (hh == 0) lse[q] = (m_ref[qb] + __log2f(lt)) * kLn2;
        }
    }
}

// ---------------------------------------------------------------------------------
// fp32 forward: every value in fp32, vector ALU only.  Two lanes share a query
// row (each holds half of d); 32 rows per wave, K/V tiles of 32 keys in LDS.
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void fa_fwd_f32_kernel(FwdParams p) {
    constexpr int KT = 32;
    constexpr int DH = D / 2;
    __shared__ __attribute__((aligned(16))) float ks[KT][D];
    __shared__ __attribute__((aligned(16))) float vs[KT][D];

    const int lane = threadIdx.x;
    const int half = lane & 1;
    const int N = p.N;
    const int ntile_q = (N + 31) / 32;
    const int head = blockIdx.x / ntile_q;
    const int qt = blockIdx.x % ntile_q;
    const int hq = head % p.Hq;
    const int b = head / p.Hq;
    const int hkv = hq / (p.Hq / p.Hkv);
    const float* Qh = (const float*)p.q + (size_t)head * N * D;
    const float* Kh = (const float*)p.k + ((size_t)b * p.Hkv + hkv) * N * D;
    const float* Vh = (const float*)p.v + ((size_t)b * p.Hkv + hkv) * N * D;
    const int q = qt * 32 + (lane >> 1);
    const bool qvalid = q < N;

    float qr[DH], acc[DH];
#pragma unroll
    for (int i = 0; i < DH; ++i) {
        qr[i] = qvalid ? Qh[(size_t)q * D + half * DH + i] : 0.f;
        acc[i] = 0.f;
    }
    float m = kNegInf, l = 0.f;
    const int q_last = min(qt * 32 + 31, N - 1);
    const int kend = p.causal ? q_last + 1 : N;

    for (int k0 = 0; k0 < kend; k0 += KT) {
        __syncthreads();
        for (int idx = lane; idx < KT * D / 4; idx += 64) {
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            const bool ok = k0 + row < N;
            ((f32x4*)ks[row])[c4] = ok ? ((const f32x4*)(Kh + (size_t)(k0 + row) * D))[c4] : f32x4{0, 0, 0, 0};
            ((f32x4*)vs[row])[c4] = ok ? ((const f32x4*)(Vh + (size_t)(k0 + row) * D))[c4] : f32x4{0, 0, 0, 0};
        }
        __syncthreads();
        float s[KT];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < DH; ++i) dot = __builtin_fmaf(qr[i], ks[j][half * DH + i], dot);
            dot += __shfl_xor(dot, 1);
            const int key = k0 + j;
            const bool vis = key < N && (!p.causal || key <= q);
            s[j] = vis ? dot * p.scale : kNegInf;
            mx = fmaxf(mx, s[j]);
        }
        const float mnew = fmaxf(m, mx);
        if (mnew != kNegInf) {
            const float alpha = m == kNegInf ? 0.f : expf(m - mnew);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < DH; ++i) acc[i] *= alpha;
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                const float pj = s[j] == kNegInf ? 0.f : expf(s[j] - mnew);
                l += pj;
#pragma unroll
                for (int i = 0; i < DH; ++i) acc[i] = __builtin_fmaf(pj, vs[j][half * DH + i], acc[i]);
            }
            m = mnew;
        }
    }
    if (qvalid) {
        float* Oh = (float*)p.o + (size_t)head * N * D;
#pragma unroll
        for (int i = 0; i < DH; ++i) Oh[(size_t)q * D + half * DH + i] = acc[i] / l;
        if (half == 0) p.lse[(size_t)head * N + q] = m + logf(l);
    }
}

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------
template <int D, int QB>
static hipError_t launch_bf16(const FwdParams& p, hipStream_t stream) {
    const int br = FwdCfg<D, QB>::BR;
    const long long nblk = (long long)p.B * p.Hq * ((p.N + br - 1) / br);
    hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, QB>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

long long fwd_bf16_grid(int B, int Hq, int N, int d) {
    const int br = d == 64 ? FwdCfg<64, kFwdQB64>::BR : FwdCfg<128, kFwdQB128>::BR;
    return (long long)B * Hq * ((N + br - 1) / br);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t stream) {
    return d == 64 ? launch_bf16<64, kFwdQB64>(p, stream) : launch_bf16<128, kFwdQB128>(p, stream);
}

long long fwd_f32_grid(int B, int Hq, int N) { return (long long)B * Hq * ((N + 31) / 32); }

hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t stream) {
    const unsigned nblk = (unsigned)fwd_f32_grid(p.B, p.Hq, p.N);
    if (d == 64)
        hipLaunchKernelGGL(fa_fwd_f32_kernel<64>, dim3(nblk), dim3(64), 0, stream, p);
    else
        hipLaunchKernelGGL(fa_fwd_f32_kernel<128>, dim3(nblk), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
