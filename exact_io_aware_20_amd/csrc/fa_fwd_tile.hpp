// Per-tile steps of the bf16 forward, shared by the full-sequence forward and the
// decode kernel: one wave, 32 query columns, one 64-key K/V tile in LDS.
//
// The method (page "LLM interview question bank" ch.029 #36, section 3, and the
// lecture summary's "推导 FlashAttention 的在线 softmax"): scores of the tile, a
// running row maximum, exponentials against it, and the rescale of the running
// output and denominator whenever the maximum moves.
#pragma once

#include "fa_common.hpp"

namespace fa {

// The reference maximum (base-2 units) moves only when a row's maximum exceeds it
// by more than this, so p <= 2^8 and the rescale is skipped on almost every tile.
constexpr float kRescaleLog2 = 8.0f;

// S^T = K Q^T for one 64-key tile and one wave's 32 queries: two 32 x 32 blocks,
// each a chain of D/16 MFMAs.  All K fragments of a 16-wide chunk pair are read
// before their MFMAs so that LDS latency overlaps the matrix pipe.
template <int D, int KMODE = 0>
__device__ __forceinline__ void fwd_scores(const uint16_t* Ks, const u32x4 (&qf)[D / 16], f32x16 (&s)[2],
                                           int l32, int hh) {
    using KT = SwzTile<D, KMODE>;
    s[0] = zero16();
    s[1] = zero16();
    constexpr int G = D / 32;   // groups of two k-chunks
#pragma unroll
    for (int g = 0; g < G; ++g) {
        u32x4 kf[2][2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) kf[cc][kb] = lds16(Ks + KT::at(32 * kb + l32, 2 * (2 * g + cc) + hh));
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(kf[cc][kb], qf[2 * g + cc], s[kb]);
    }
}

// fwd_scores in a scheduling region of its own: the two 32-key chains taken in turn,
// one K fragment per MFMA read two MFMAs ahead (a ring of three); same accumulation
// order as fwd_scores.
template <int D>
__device__ __forceinline__ void fwd_scores_ring(const uint16_t* Ks, const u32x4 (&qf)[D / 16], f32x16 (&s)[2],
                                                int l32, int hh) {
    using KT = SwzTile<D, 0>;
    constexpr int M = D / 8;   // m: chunk m / 2 of key block m % 2
    auto frag = [&](int m) __attribute__((always_inline)) { return lds16(Ks + KT::at(32 * (m & 1) + l32, 2 * (m >> 1) + hh)); };
    __builtin_amdgcn_sched_barrier(0);
    s[0] = zero16();
    s[1] = zero16();
    u32x4 a[3];
    a[0] = frag(0);
    a[1] = frag(1);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (m + 2 < M) a[(m + 2) % 3] = frag(m + 2);
        s[m & 1] = mfma32x32x16(a[m % 3], qf[m >> 1], s[m & 1]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // reads of MFMAs 0 and 1
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (m + 2 < M) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // read of MFMA m+2
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA m
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Max over the wave's lane pair (l, l^32) that share a query column.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Keys outside [lo, hi], this lane's visible band (hi already clipped below N; lo
// checked only when LO): masked scores become -inf (p = 0).
template <bool LO>
__device__ __forceinline__ void fwd_mask(f32x16 (&s)[2], int k0, int lo, int hi, int hh) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool vis = key <= hi && (!LO || key >= lo);
            s[kb][r] = vis ? s[kb][r] : kNegInf;
        }
}

// Row max (in-lane chain, then the partner lane) and the lazy rescale: the
// reference m_ref (base-2 units) moves only when the row maximum exceeds it by
// more than kRescaleLog2; O and l are then multiplied by 2^(m_old - m_new).
template <int D>
__device__ __forceinline__ void fwd_rescale(const f32x16 (&s)[2], f32x16 (&o)[D / 32], float& m_ref, float& l_part,
                                            float sl2) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair_max(mx);
    const float mt = mx * sl2;   // sl2 > 0, so -inf stays -inf
    const bool need = mt > m_ref + kRescaleLog2;
    if (__builtin_expect(__ballot(need) != 0, 0)) {
        const float mnew = need ? mt : m_ref;
        const float alpha = m_ref == kNegInf ? 0.f : fast_exp2(m_ref - mnew);
        m_ref = mnew;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
}

// P = 2^(S*sl2 - m_ref), rounded to bf16 and packed as the B operand of
// O^T = V^T P^T; l accumulates the same rounded values.
__device__ __forceinline__ void fwd_probs(const f32x16 (&s)[2], float m_ref, float sl2, u32x4 (&pf)[2][2],
                                          float& l_part) {
    const float mref = m_ref == kNegInf ? 0.f : m_ref;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float pa = fast_exp2(__builtin_fmaf(s[kb][8 * h2 + 2 * j], sl2, -mref));
                const float pb = fast_exp2(__builtin_fmaf(s[kb][8 * h2 + 2 * j + 1], sl2, -mref));
                const uint32_t pk = pack_bf16(pa, pb);
                pf[kb][h2][j] = pk;
                l_part = add_bf16_pair(pk, l_part);
            }
}

// O^T += V^T P^T over the tile's 64 keys (A operand read transposed from the
// natural V tile).
template <int D>
__device__ __forceinline__ void fwd_pv(const uint16_t* Vt, const u32x4 (&pf)[2][2], f32x16 (&o)[D / 32], int lane) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                o[db] = mfma32x32x16(tr_frag<D>(Vt, db, 32 * kb + 16 * h2, lane), pf[kb][h2], o[db]);
}

// fwd_pv in a scheduling region of its own: the transposed V fragments read three
// MFMAs ahead (a ring of four), so that an MFMA's operand is never the youngest read in
// flight.  Same accumulation order as fwd_pv.
template <int D>
__device__ __forceinline__ void fwd_pv_ring(const uint16_t* Vt, const u32x4 (&pf)[2][2], f32x16 (&o)[D / 32],
                                            int lane) {
    constexpr int DB = D / 32;
    constexpr int M = 4 * DB;   // m: column block m % DB of (kb, h2) = (m / DB) / 2, (m / DB) % 2
    auto frag = [&](int m) __attribute__((always_inline)) {
        const int kh = m / DB;
        return tr_frag<D>(Vt, m % DB, 32 * (kh >> 1) + 16 * (kh & 1), lane);
    };
    __builtin_amdgcn_sched_barrier(0);
    u32x4 a[4];
#pragma unroll
    for (int m = 0; m < 3; ++m) a[m] = frag(m);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (m + 3 < M) a[(m + 3) & 3] = frag(m + 3);
        const int kh = m / DB;
        o[m % DB] = mfma32x32x16(a[m & 3], pf[kh >> 1][kh & 1], o[m % DB]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // reads of MFMAs 0-2
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (m + 3 < M) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // reads of MFMA m+3
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA m
    }
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace fa
