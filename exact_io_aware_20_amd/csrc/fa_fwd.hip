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
//   * 8 waves per workgroup (two per SIMD, so one wave's softmax overlaps the
//     other's matrix work), each owning 32 query rows.  K/V tiles of 64 keys are
//     double-buffered in LDS with one barrier per tile; both arrive by direct
//     global->LDS loads into XOR-swizzled natural layouts (no register staging).
//   * Scores are formed transposed, S^T = K Q^T, so a lane holds one query (its
//     column) and 16 keys; the row maximum is an in-lane max plus one exchange
//     with lane l^32, and the running statistics are lane-local scalars.
//   * O^T = V^T P^T reuses the S^T registers, rounded to bf16, directly as the
//     B operand; the V^T A operand is read from the natural V tile with the
//     transposing LDS read (two 8-byte reads per fragment).
//   * Scores are kept in base-2 units (scale*log2 e folded into one FMA before
//     v_exp_f32).  The reference maximum is only moved when a row's maximum
//     grows by more than 2^8 (kRescaleLog2): the quotient O = sum p v / sum p is
//     the same for any reference, p stays <= 256, and the O rescale, which costs
//     d/64 multiplies per score, is skipped on almost every tile.
//   * Masks: every tile bound and mask test is written through the visible band
//     (key j visible to query i iff i - wl <= j <= i + wr), so the causal, full and
//     sliding-window forms share one kernel (the window form in its own
//     instantiation); block-sparse layouts use the list-driven kernel further down.
#include "fa_common.hpp"
#include "fa_fwd_tile.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
struct FwdCfg {
    static constexpr int WAVES = 8;               // two waves per SIMD
    static constexpr int THREADS = WAVES * kWave;
    static constexpr int BR = WAVES * 32;         // query rows per workgroup (32 per wave)
    static constexpr int BC = 64;                 // keys per K/V tile
    static constexpr int DC = D / 16;             // k-chunks of the S contraction
    static constexpr int DB = D / 32;             // 32-row blocks of O^T
    // K/V tile loads in the buffer form (exact LDS waits under in-flight loads); at
    // d = 64 the global form measured about 1 % faster
    static constexpr bool BUF_DMA = D > 64;
    static_assert(BR == kFwdRows, "launch plan and kernel disagree on the row tile");
};

// Loop-hoisted LDS addressing of the K fragments: the swizzle depends on the row mod
// 16 only, so fragment (kb, chunk c) of lane l sits at a per-lane byte offset for c
// plus the constant 32 kb rows.  A step adds its buffer's base to the D/16 offsets
// once (hidden from the optimiser) and every read keeps its constant as an
// immediate.  The window instantiation uses this addressing (with the V tile read
// through TrAddr): its first tile index is not known at compile time, and with
// plain pointers the compiler kept per-buffer copies of every fragment address and
// spilled; the addressing measured 6 % faster there and ≈ 1 % slower without a window.
template <int D>
struct KFragAddr {
    uint32_t a[D / 16];
    __device__ __forceinline__ KFragAddr(const uint32_t (&off)[D / 16], uint32_t base) {
#pragma unroll
        for (int c = 0; c < D / 16; ++c) a[c] = opaque(base + off[c]);
    }
};
template <int D>
__device__ __forceinline__ void kfrag_offsets(uint32_t (&off)[D / 16], int l32, int hh) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) off[c] = 2u * (uint32_t)SwzTile<D, 0>::at(l32, 2 * c + hh);
}

// fwd_scores with the K tile addressed through KFragAddr
template <int D>
__device__ __forceinline__ void fwd_scores_a(const KFragAddr<D>& ka, const u32x4 (&qf)[D / 16], f32x16 (&s)[2]) {
    s[0] = zero16();
    s[1] = zero16();
    constexpr int G = D / 32;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        u32x4 kf[2][2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) kf[cc][kb] = lds16_a(ka.a[2 * g + cc] + kb * 2 * 32 * D);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(kf[cc][kb], qf[2 * g + cc], s[kb]);
    }
}

// fwd_pv with the V tile addressed through TrAddr
template <int D>
__device__ __forceinline__ void fwd_pv_a(const TrAddr<D>& va, const u32x4 (&pf)[2][2], f32x16 (&o)[D / 32]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] = mfma32x32x16(va.frag(db, 32 * kb + 16 * h2), pf[kb][h2], o[db]);
}

// fwd_pv_a in a scheduling region of its own, the transposed V fragments read three
// MFMAs ahead (a ring of four); same accumulation order.
template <int D>
__device__ __forceinline__ void fwd_pv_a_ring(const TrAddr<D>& va, const u32x4 (&pf)[2][2], f32x16 (&o)[D / 32]) {
    constexpr int DB = D / 32;
    constexpr int M = 4 * DB;   // m: column block m % DB of (kb, h2) = (m / DB) / 2, (m / DB) % 2
    auto frag = [&](int m) __attribute__((always_inline)) {
        const int kh = m / DB;
        return va.frag(m % DB, 32 * (kh >> 1) + 16 * (kh & 1));
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

// Epilogue store of one query row (row index `row` of [B*Hq*N]): the lane's O^T
// registers times inv = 1/l, rounded to bf16 (round to nearest even).  With the
// validation pointer p.o32 set, the same fp32 products are stored unrounded instead.
template <int D>
__device__ __forceinline__ void store_o(const FwdParams& p, size_t row, const f32x16 (&o)[D / 32], float inv,
                                        int hh) {
    if (p.o32) {
        float* Or = p.o32 + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(f32x4*)(Or + 32 * db + 8 * g + 4 * hh) =
                    f32x4{o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
        return;
    }
    uint16_t* Or = (uint16_t*)p.o + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x2 v2 = {pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                              pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
            *(u32x2*)(Or + 32 * db + 8 * g + 4 * hh) = v2;
        }
}

// The kernel is software-pipelined by one tile: S(t+1) = K(t+1) Q^T goes to the
// matrix cores while the vector units turn S(t) into probabilities.  LDS holds
// K(t+1) and V(t) during step t; the direct loads of K(t+2) and V(t+1) fill the
// other halves of the two double buffers meanwhile, one workgroup barrier per step.
// The leading steps, whose current and next tiles are fully visible to every row
// of the workgroup, run as branch-free blocks in a loop of their own; the
// diagonal and ragged tail steps take the general path.
template <int D, bool WINDOW>
__global__ __launch_bounds__(FwdCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_kernel(FwdParams p) {
    using C = FwdCfg<D>;
    constexpr int KB = SwzTile<D, 0>::ELEMS;
    constexpr int VB = SwzTile<D, 1>::ELEMS;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KB + 2 * VB];
    uint16_t* kbuf = smem;            // K tile of parity t&1 at kbuf + (t&1)*KB
    uint16_t* vbuf = smem + 2 * KB;   // V tile of parity t&1 at vbuf + (t&1)*VB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave < C::WAVES);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = p.N;
    // Visible band: key j is visible to query i iff i - wl <= j <= i + wr (and j < N).
    // Without a window wl = N (no lower limit); causal means wr = 0.
    const int wl = WINDOW ? p.window : N;
    const int wr = p.causal ? 0 : (WINDOW ? p.window : N);

    const int ntile_q = (N + C::BR - 1) / C::BR;
    int head, qt;
    map_block(blockIdx.x, gridDim.x, ntile_q, p.B * p.Hq, p.causal != 0, head, qt, 4);
    const int hq = head % p.Hq;
    const int b = head / p.Hq;
    const int hkv = hq / (p.Hq / p.Hkv);

    const uint16_t* Qh = (const uint16_t*)p.q + (size_t)head * N * D;
    const uint16_t* Kh = (const uint16_t*)p.k + ((size_t)b * p.Hkv + hkv) * N * D;
    const uint16_t* Vh = (const uint16_t*)p.v + ((size_t)b * p.Hkv + hkv) * N * D;

    const int q0 = qt * C::BR;
    const int qw0 = q0 + wave * 32;
    const int q = qw0 + l32;
    const int q_last = min(q0 + C::BR, N) - 1;
    // tiles [t_begin, ntiles) hold a key visible to some row of the workgroup
    const int t_begin = WINDOW ? max(0, q0 - wl) / C::BC : 0;
    const int ntiles = min(N - 1, q_last + wr) / C::BC + 1;
    const int wq_last = min(qw0 + 32, N) - 1;
    const int wave_tiles = wq_last < qw0 ? 0 : min(N - 1, wq_last + wr) / C::BC + 1;

    // Q fragments: B operand of S^T = K Q^T (lane: query, slots: 8 consecutive d).
    u32x4 qf[C::DC];
#pragma unroll
    for (int c = 0; c < C::DC; ++c)
        qf[c] = q < N ? ld_global16(Qh + (size_t)q * D + 16 * c + 8 * hh) : zero_u4();

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = zero16();
    float m_ref = kNegInf, l_part = 0.f;
    const float sl2 = p.scale_log2;

    TileDma<D, 0, C::WAVES, C::BUF_DMA> kdma;
    TileDma<D, 1, C::WAVES, C::BUF_DMA> vdma;
    kdma.init(wave, lane);
    vdma.init(wave, lane);
    auto issue_k = [&](int t, uint16_t* buf) { kdma.issue(Kh + (size_t)t * C::BC * D, N - t * C::BC, buf, wave); };
    auto issue_v = [&](int t, uint16_t* buf) { vdma.issue(Vh + (size_t)t * C::BC * D, N - t * C::BC, buf, wave); };

    uint32_t koff[C::DC];
    TrOffsets<D> voff;
    if constexpr (WINDOW) {
        kfrag_offsets<D>(koff, l32, hh);
        voff.init(lane);
    }
    // S^T of the K tile in `buf`, and O^T += V^T P^T with the V tile in `buf`
    auto scores_of = [&](const uint16_t* buf, f32x16 (&dst)[2]) {
        if constexpr (WINDOW) {
            const KFragAddr<D> ka(koff, lds_addr(buf));
            fwd_scores_a<D>(ka, qf, dst);
        } else {
            fwd_scores<D>(buf, qf, dst, l32, hh);
        }
    };
    auto pv_of = [&](const uint16_t* buf, const u32x4 (&pf)[2][2]) {
        if constexpr (WINDOW) {
            const TrAddr<D> va(voff, lds_addr(buf));
            fwd_pv_a<D>(va, pf, o);
        } else {
            fwd_pv_ring<D>(buf, pf, o, lane);
        }
    };

    // prologue: K(t0), V(t0) and K(t0+1) -> LDS in one round trip (buffers by tile
    // parity); S(t0); a barrier before the first step reloads K(t0)'s buffer
    const int tb = t_begin & 1;
    issue_k(t_begin, kbuf + tb * KB);
    issue_v(t_begin, vbuf + tb * VB);
    if (t_begin + 1 < ntiles) issue_k(t_begin + 1, kbuf + (tb ^ 1) * KB);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sa[2], sb[2];
    if (t_begin < wave_tiles) scores_of(kbuf + tb * KB, sa);
    __syncthreads();

    // Fast step: tiles t and t+1 are fully visible to every row of the workgroup
    // (so t+1 < ntiles and V(t+1) exists; K(t+2) may not, and then the last tile
    // is reloaded into the free buffer).  One branch-free block apart from the
    // rare rescale: scores(t+1) on the matrix cores interleaved with the
    // exponentials of tile t in a fixed pattern, then PV(t) (the compiler's own
    // interleave of all three phases measured slower).
    auto fast_step = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        fwd_rescale<D>(cur, o, m_ref, l_part, sl2);
        issue_k(min(t + 2, ntiles - 1), kbuf + (t & 1) * KB);
        issue_v(t + 1, vbuf + ((t + 1) & 1) * VB);
        u32x4 pf[2][2];
        // The wave in the mixed block below takes issue priority over its SIMD partner
        // in the PV block, so the partner's PV MFMAs fill the gaps between this wave's
        // exponentials (measured 0.2-0.7 % faster than equal priorities).
        __builtin_amdgcn_s_setprio(3);
        scores_of(kbuf + ((t + 1) & 1) * KB, nxt);
        fwd_probs(cur, m_ref, sl2, pf, l_part);
        // Interleave the two in one instruction stream: six K-fragment reads ahead,
        // then per score MFMA (independent of tile t's softmax) six of its vector
        // instructions and the next fragment read, so the vector work issues while
        // the matrix pipe is busy (≈ 3 % faster than the two blocks in sequence; six
        // vector instructions per MFMA measured 0.3-1.4 % faster than four on the
        // long-context forward, three and eight slower; six reads ahead 1-1.5 %
        // faster than four, two no better).
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // DS reads
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
            if (i < D / 8 - 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        pv_of(vbuf + (t & 1) * VB, pf);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // General step (diagonal and ragged tiles): tile t's softmax/PV with scores
    // `cur`, tile t+1's scores into `nxt`.
    auto step = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        const int k0 = t * C::BC;
        if (t + 2 < ntiles) issue_k(t + 2, kbuf + (t & 1) * KB);
        if (t + 1 < ntiles) issue_v(t + 1, vbuf + ((t + 1) & 1) * VB);
        if (t + 1 < wave_tiles) scores_of(kbuf + ((t + 1) & 1) * KB, nxt);
        if (t < wave_tiles) {
            if (k0 + C::BC - 1 > qw0 + wr || k0 + C::BC > N || (WINDOW && k0 < wq_last - wl))
                fwd_mask<WINDOW>(cur, k0, q - wl, min(q + wr, N - 1), hh);
            fwd_rescale<D>(cur, o, m_ref, l_part, sl2);
            u32x4 pf[2][2];
            fwd_probs(cur, m_ref, sl2, pf, l_part);
            pv_of(vbuf + (t & 1) * VB, pf);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // Keys [lo_all, hi_all] are visible to every row of the workgroup, so tiles
    // [full_lo, full_hi) are fully visible; a fast step needs tiles t and t+1 in that
    // range.  Steps before it (the band's left edge) and after it (the diagonal, the
    // band's right edge, the ragged tail) take the general path.
    const int lo_all = WINDOW ? max(0, q_last - wl) : 0;
    const int hi_all = min(N - 1, q0 + wr);
    const int full_lo = (lo_all + C::BC - 1) / C::BC;
    const int full_hi = (hi_all + 1) / C::BC;
    const int lead_end = WINDOW ? min(max(t_begin, full_lo), ntiles) : t_begin;
    const int nfast = max(lead_end, min(full_hi, ntiles) - 1);
    int t = t_begin;
    if constexpr (WINDOW) {
        for (; t + 1 < lead_end; t += 2) {
            step(t, sa, sb);
            step(t + 1, sb, sa);
        }
        if (t < lead_end) {
            step(t, sa, sb);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sa[kb] = sb[kb];
            ++t;
        }
    }
    for (; t + 1 < nfast; t += 2) {
        fast_step(t, sa, sb);
        fast_step(t + 1, sb, sa);
    }
    if (t < nfast) {
        fast_step(t, sa, sb);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sa[kb] = sb[kb];
        ++t;
    }
    // one general step per iteration, the scores handed over by copy: unrolled by two
    // (swapping the two score sets) the loop spilled 8 registers to scratch
    for (; t < ntiles; ++t) {
        step(t, sa, sb);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sa[kb] = sb[kb];
    }

    // ---- epilogue: O = O^T / l (bf16, round to nearest even), LSE in natural log
    const float lt = l_part + __shfl_xor(l_part, 32);
    if (q < N) {
        store_o<D>(p, (size_t)head * N + q, o, 1.0f / lt, hh);
        if (hh == 0) p.lse[(size_t)head * N + q] = (m_ref + __log2f(lt)) * kLn2;
    }
}

// ---------------------------------------------------------------------------------
// Persistent form of the dense forward.  The grid holds at most one workgroup per CU,
// and each walks a fixed list of (head, row tile) items (FwdSchedule).  The last step
// of an item also issues the next item's Q loads and the direct loads of its first two
// K tiles and first V tile, and the item's O and LSE are stored after that step's
// barrier, so a workgroup moves to its next item without an exposed memory round
// trip, store drain or launch gap.  Tile buffers are chosen by (t + ph) & 1 with a
// per-item parity ph, so the next item's first V tile lands in the buffer the last
// step does not read; K and V^T fragments are addressed through per-lane offsets and
// an opaque per-step base (KFragAddr, TrAddr), as the parity is not known at compile
// time.
// ---------------------------------------------------------------------------------
struct FwdSchedule {
    int M, S, x, c;
    __device__ __forceinline__ FwdSchedule(int bid, int nblk, int nitems, int nhead) {
        const int nx = ((nitems & 7) == 0 && (nhead & 7) == 0 && (nblk & 7) == 0) ? 8 : 1;
        M = nitems / nx;
        S = nblk / nx;
        x = bid % nx;
        c = bid / nx;
    }
    // logical item of round r (snake order over the S slots of an XCD), or -1
    __device__ __forceinline__ int item(int r) const {
        const int j = r * S + ((r & 1) ? S - 1 - c : c);
        return j < M ? x * M + j : -1;
    }
};

template <int D, bool WINDOW>
__global__ __launch_bounds__(FwdCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_persist_kernel(FwdParams p) {
    using C = FwdCfg<D>;
    constexpr int KB = SwzTile<D, 0>::ELEMS;
    constexpr int VB = SwzTile<D, 1>::ELEMS;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KB + 2 * VB];
    uint16_t* kbuf = smem;
    uint16_t* vbuf = smem + 2 * KB;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave < C::WAVES);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = p.N;
    const int wl = WINDOW ? p.window : N;
    const int wr = p.causal ? 0 : (WINDOW ? p.window : N);

    const int ntile_q = (N + C::BR - 1) / C::BR;
    const int nhead = p.B * p.Hq;
    const FwdSchedule sched(blockIdx.x, gridDim.x, nhead * ntile_q, nhead);
    int item = sched.item(0);
    if (item < 0) return;

    struct Geom {
        int head, q0, qw0, q_last, wq_last, t_begin, ntiles, wave_tiles;
        const uint16_t *Qh, *Kh, *Vh;
    };
    auto geom = [&](int it) __attribute__((always_inline)) {
        Geom g;
        int qt;
        decode_item(it, ntile_q, nhead, p.causal != 0, g.head, qt, 4);
        const int hq = g.head % p.Hq;
        const int b = g.head / p.Hq;
        const int hkv = hq / (p.Hq / p.Hkv);
        g.Qh = (const uint16_t*)p.q + (size_t)g.head * N * D;
        g.Kh = (const uint16_t*)p.k + ((size_t)b * p.Hkv + hkv) * N * D;
        g.Vh = (const uint16_t*)p.v + ((size_t)b * p.Hkv + hkv) * N * D;
        g.q0 = qt * C::BR;
        g.qw0 = g.q0 + wave * 32;
        g.q_last = min(g.q0 + C::BR, N) - 1;
        g.t_begin = WINDOW ? max(0, g.q0 - wl) / C::BC : 0;
        g.ntiles = min(N - 1, g.q_last + wr) / C::BC + 1;
        g.wq_last = min(g.qw0 + 32, N) - 1;
        g.wave_tiles = g.wq_last < g.qw0 ? 0 : min(N - 1, g.wq_last + wr) / C::BC + 1;
        return g;
    };

    TileDma<D, 0, C::WAVES, C::BUF_DMA> kdma;
    TileDma<D, 1, C::WAVES, C::BUF_DMA> vdma;
    kdma.init(wave, lane);
    vdma.init(wave, lane);
    auto issue_k = [&](const Geom& g, int t, uint16_t* buf) __attribute__((always_inline)) {
        kdma.issue(g.Kh + (size_t)t * C::BC * D, N - t * C::BC, buf, wave);
    };
    auto issue_v = [&](const Geom& g, int t, uint16_t* buf) __attribute__((always_inline)) {
        vdma.issue(g.Vh + (size_t)t * C::BC * D, N - t * C::BC, buf, wave);
    };
    uint32_t koff[C::DC];
    kfrag_offsets<D>(koff, l32, hh);
    TrOffsets<D> voff;
    voff.init(lane);

    u32x4 qf[C::DC];
    f32x16 o[C::DB];
    auto scores_of = [&](const uint16_t* buf, f32x16 (&dst)[2]) __attribute__((always_inline)) {
        const KFragAddr<D> ka(koff, lds_addr(buf));
        fwd_scores_a<D>(ka, qf, dst);
    };
    auto pv_of = [&](const uint16_t* buf, const u32x4 (&pf)[2][2]) __attribute__((always_inline)) {
        const TrAddr<D> va(voff, lds_addr(buf));
        fwd_pv_a_ring<D>(va, pf, o);
    };
    // an item's Q fragments, first two K tiles and first V tile (buffer parity ph)
    auto prefetch = [&](const Geom& g, int ph) __attribute__((always_inline)) {
        const int qq = g.qw0 + l32;
#pragma unroll
        for (int c = 0; c < C::DC; ++c)
            qf[c] = qq < N ? ld_global16(g.Qh + (size_t)qq * D + 16 * c + 8 * hh) : zero_u4();
        issue_k(g, g.t_begin, kbuf + ((g.t_begin + ph) & 1) * KB);
        issue_v(g, g.t_begin, vbuf + ((g.t_begin + ph) & 1) * VB);
        if (g.t_begin + 1 < g.ntiles) issue_k(g, g.t_begin + 1, kbuf + ((g.t_begin + 1 + ph) & 1) * KB);
    };

    Geom cur = geom(item);
    int ph = 0;
    prefetch(cur, ph);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    float m_ref, l_part;
    const float sl2 = p.scale_log2;
    for (int r = 0;;) {
        const int q = cur.qw0 + l32;
        const int qw0 = cur.qw0, wq_last = cur.wq_last, ntiles = cur.ntiles, wave_tiles = cur.wave_tiles;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] = zero16();
        m_ref = kNegInf;
        l_part = 0.f;

        f32x16 sa[2], sb[2];
        if (cur.t_begin < wave_tiles) scores_of(kbuf + ((cur.t_begin + ph) & 1) * KB, sa);
        __syncthreads();   // K(t_begin) read by every wave: its buffer takes K(t_begin + 2)

        auto fast_step = [&](int t, f32x16 (&cs)[2], f32x16 (&ns)[2]) __attribute__((always_inline)) {
            fwd_rescale<D>(cs, o, m_ref, l_part, sl2);
            issue_k(cur, min(t + 2, ntiles - 1), kbuf + ((t + ph) & 1) * KB);
            issue_v(cur, t + 1, vbuf + ((t + 1 + ph) & 1) * VB);
            u32x4 pf[2][2];
            scores_of(kbuf + ((t + 1 + ph) & 1) * KB, ns);
            fwd_probs(cs, m_ref, sl2, pf, l_part);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < D / 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                if (i < D / 8 - 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            pv_of(vbuf + ((t + ph) & 1) * VB, pf);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        auto finish_tile = [&](int t, f32x16 (&cs)[2]) __attribute__((always_inline)) {
            const int k0 = t * C::BC;
            if (k0 + C::BC - 1 > qw0 + wr || k0 + C::BC > N || (WINDOW && k0 < wq_last - wl))
                fwd_mask<WINDOW>(cs, k0, q - wl, min(q + wr, N - 1), hh);
            fwd_rescale<D>(cs, o, m_ref, l_part, sl2);
            u32x4 pf[2][2];
            fwd_probs(cs, m_ref, sl2, pf, l_part);
            pv_of(vbuf + ((t + ph) & 1) * VB, pf);
        };
        auto step = [&](int t, f32x16 (&cs)[2], f32x16 (&ns)[2]) __attribute__((always_inline)) {
            if (t + 2 < ntiles) issue_k(cur, t + 2, kbuf + ((t + ph) & 1) * KB);
            issue_v(cur, t + 1, vbuf + ((t + 1 + ph) & 1) * VB);
            if (t + 1 < wave_tiles) scores_of(kbuf + ((t + 1 + ph) & 1) * KB, ns);
            if (t < wave_tiles) finish_tile(t, cs);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        int t = cur.t_begin;
        auto general_steps = [&](int end) __attribute__((always_inline)) {
            for (; t + 1 < end; t += 2) {
                step(t, sa, sb);
                step(t + 1, sb, sa);
            }
            if (t < end) {
                step(t, sa, sb);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) sa[kb] = sb[kb];
                ++t;
            }
        };
        const int lo_all = WINDOW ? max(0, cur.q_last - wl) : 0;
        const int hi_all = min(N - 1, cur.q0 + wr);
        const int full_lo = (lo_all + C::BC - 1) / C::BC;
        const int full_hi = (hi_all + 1) / C::BC;
        const int lead_end = WINDOW ? min(max(cur.t_begin, full_lo), ntiles - 1) : cur.t_begin;
        const int nfast = min(ntiles - 1, max(lead_end, min(full_hi, ntiles) - 1));
        if constexpr (WINDOW) general_steps(lead_end);
        for (; t + 1 < nfast; t += 2) {
            fast_step(t, sa, sb);
            fast_step(t + 1, sb, sa);
        }
        if (t < nfast) {
            fast_step(t, sa, sb);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sa[kb] = sb[kb];
            ++t;
        }
        general_steps(ntiles - 1);

        // last step (t = ntiles - 1): the next item's loads go out first
        const int nitem = sched.item(++r);
        Geom nxt = cur;
        int nph = ph;
        if (nitem >= 0) {
            nxt = geom(nitem);
            nph = (t + ph + 1 - nxt.t_begin) & 1;
            prefetch(nxt, nph);
        }
        if (t < wave_tiles) finish_tile(t, sa);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        // epilogue of the finished item: O = O^T / l (bf16, RNE), LSE in natural log
        const float lt = l_part + __shfl_xor(l_part, 32);
        if (q < N) {
            store_o<D>(p, (size_t)cur.head * N + q, o, 1.0f / lt, hh);
            if (hh == 0) p.lse[(size_t)cur.head * N + q] = (m_ref + __log2f(lt)) * kLn2;
        }
        if (nitem < 0) break;
        cur = nxt;
        ph = nph;
    }
}

// ---------------------------------------------------------------------------------
// Block-sparse forward (page "ZeRO 与 FlashAttention 各优化什么?", section
// "注意力瓶颈与优化路线": block-sparse patterns compute only part of the positions).
// The workgroup's 256 rows are four 64-row blocks of the layout; wave 0 compacts the
// key tiles that any of them sees (layout bit set, and not after the block under the
// causal rule) into an LDS list, tagged with which blocks see each, and the workgroup
// walks that list with the per-tile steps above, pipelined by one entry like the dense
// kernel (K/V double-buffered, one barrier per entry); a wave computes only the tiles
// its own block sees.  A row that sees no key gets O = 0 and LSE = -inf.
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(FwdCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_sparse_kernel(FwdParams p) {
    using C = FwdCfg<D>;
    constexpr int KB = SwzTile<D, 0>::ELEMS;
    constexpr int VB = SwzTile<D, 1>::ELEMS;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KB + 2 * VB];
    __shared__ uint32_t list[kSparseMaxBlocks];
    __shared__ int list_n;
    uint16_t* kbuf = smem;
    uint16_t* vbuf = smem + 2 * KB;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave < C::WAVES);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = p.N;
    const int wr = p.causal ? 0 : N;

    const int ntile_q = (N + C::BR - 1) / C::BR;
    int head, qt;
    map_block(blockIdx.x, gridDim.x, ntile_q, p.B * p.Hq, p.causal != 0, head, qt, 4);
    const int hq = head % p.Hq;
    const int b = head / p.Hq;
    const int hkv = hq / (p.Hq / p.Hkv);
    const uint16_t* Qh = (const uint16_t*)p.q + (size_t)head * N * D;
    const uint16_t* Kh = (const uint16_t*)p.k + ((size_t)b * p.Hkv + hkv) * N * D;
    const uint16_t* Vh = (const uint16_t*)p.v + ((size_t)b * p.Hkv + hkv) * N * D;

    const int q0 = qt * C::BR;
    const int qw0 = q0 + wave * 32;
    const int q = qw0 + l32;
    const int nb = (N + kSparseBlock - 1) / kSparseBlock;
    const int qb0 = q0 / kSparseBlock;
    // Q fragments first, so that their loads are in flight with the layout reads of
    // the list build (B operand of S^T = K Q^T, lane: query)
    u32x4 qf[C::DC];
#pragma unroll
    for (int c = 0; c < C::DC; ++c)
        qf[c] = q < N ? ld_global16(Qh + (size_t)q * D + 16 * c + 8 * hh) : zero_u4();
    if (wave == 0) {
        const int u_end = p.causal ? min(nb, qb0 + C::BR / kSparseBlock) : nb;   // later key tiles are masked
        const int n = compact_tiles(list, 0, u_end, lane, [&](int u) -> uint32_t {
            uint32_t bits = 0;
#pragma unroll
            for (int j = 0; j < C::BR / kSparseBlock; ++j) {
                const int qb = qb0 + j;
                const bool set = p.block_mask[(size_t)min(qb, nb - 1) * nb + u] != 0;
                bits |= (uint32_t)((qb < nb) & (!p.causal | (u <= qb)) & set) << j;
            }
            return bits;
        });
        if (lane == 0) list_n = n;
    }
    __syncthreads();
    const int cnt = list_n;
    const int wbit = 20 + wave / (kSparseBlock / 32);   // this wave's block within the workgroup

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = zero16();
    float m_ref = kNegInf, l_part = 0.f;
    const float sl2 = p.scale_log2;

    TileDma<D, 0, C::WAVES, C::BUF_DMA> kdma;
    TileDma<D, 1, C::WAVES, C::BUF_DMA> vdma;
    kdma.init(wave, lane);
    vdma.init(wave, lane);
    auto tile = [&](int e) { return (int)(list[e] & kSparseTileMask); };
    auto sees = [&](int e) { return ((list[e] >> wbit) & 1u) && qw0 < N; };
    auto issue_k = [&](int e, uint16_t* buf) {
        const int t = tile(e);
        kdma.issue(Kh + (size_t)t * C::BC * D, N - t * C::BC, buf, wave);
    };
    auto issue_v = [&](int e, uint16_t* buf) {
        const int t = tile(e);
        vdma.issue(Vh + (size_t)t * C::BC * D, N - t * C::BC, buf, wave);
    };

    // Software-pipelined like the dense kernel, over list entries: step e forms the
    // scores of entry e+1 (if this wave's block sees it) while it runs the softmax
    // and P.V of entry e; LDS holds K(e+1) and V(e) during step e, and the loads of
    // K(e+2) and V(e+1) fill the other halves of the two double buffers.
    f32x16 sa[2], sb[2];
    if (cnt > 0) {   // K(0), V(0) and K(1) in one round trip, as in the dense kernel
        issue_k(0, kbuf);
        issue_v(0, vbuf);
        if (1 < cnt) issue_k(1, kbuf + KB);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (sees(0)) fwd_scores_ring<D>(kbuf, qf, sa, l32, hh);
        __syncthreads();
    }
    auto step = [&](int e, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        if (e + 2 < cnt) issue_k(e + 2, kbuf + (e & 1) * KB);
        if (e + 1 < cnt) issue_v(e + 1, vbuf + ((e + 1) & 1) * VB);
        if (e + 1 < cnt && sees(e + 1)) fwd_scores_ring<D>(kbuf + ((e + 1) & 1) * KB, qf, nxt, l32, hh);
        if (sees(e)) {
            const int k0 = tile(e) * C::BC;
            if (k0 + C::BC - 1 > qw0 + wr || k0 + C::BC > N) fwd_mask<false>(cur, k0, 0, min(q + wr, N - 1), hh);
            fwd_rescale<D>(cur, o, m_ref, l_part, sl2);
            u32x4 pf[2][2];
            fwd_probs(cur, m_ref, sl2, pf, l_part);
            fwd_pv_ring<D>(vbuf + (e & 1) * VB, pf, o, lane);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    for (int e = 0; e < cnt; e += 2) {
        step(e, sa, sb);
        if (e + 1 < cnt) step(e + 1, sb, sa);
    }

    const float lt = l_part + __shfl_xor(l_part, 32);
    if (q < N) {
        const bool any = lt > 0.f;
        uint16_t* Oh = (uint16_t*)p.o + (size_t)head * N * D + (size_t)q * D;
        const float inv = any ? 1.0f / lt : 0.f;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2 v2 = {pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                  pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
                *(u32x2*)(Oh + 32 * db + 8 * g + 4 * hh) = v2;
            }
        if (hh == 0) p.lse[(size_t)head * N + q] = any ? (m_ref + __log2f(lt)) * kLn2 : kNegInf;
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
template <int D>
static hipError_t launch_bf16(const FwdParams& p, hipStream_t stream) {
    constexpr int br = FwdCfg<D>::BR;
    const long long nblk = (long long)p.B * p.Hq * ((p.N + br - 1) / br);
    if (p.block_mask)
        hipLaunchKernelGGL((fa_fwd_sparse_kernel<D>), dim3((unsigned)nblk), dim3(FwdCfg<D>::THREADS), 0, stream, p);
    else if (p.window < 0 && D == 128) {
        // dense d = 128: the non-persistent kernel measured 1.5-2 % faster (its direct
        // fragment addressing and dynamic workgroup dispatch outweigh the fixed cost the
        // persistent form hides at these tile counts)
        if constexpr (D == 128)
            hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, false>), dim3((unsigned)nblk), dim3(FwdCfg<D>::THREADS), 0,
                               stream, p);
    } else {
        // sliding window (4 % faster persistent) and d = 64 (2 % faster): one workgroup
        // per compute unit of the device the stream belongs to
        int dev = 0, ncu = 0;
        hipError_t e = hipStreamGetDevice(stream, &dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (ncu < 1) return hipErrorInvalidDevice;
        const long long nhead = (long long)p.B * p.Hq;
        long long grid = nblk < ncu ? nblk : ncu;
        if ((nblk & 7) == 0 && (nhead & 7) == 0 && grid >= 8) grid -= grid & 7;
        if (p.window >= 0)
            hipLaunchKernelGGL((fa_fwd_persist_kernel<D, true>), dim3((unsigned)grid), dim3(FwdCfg<D>::THREADS), 0,
                               stream, p);
        else if constexpr (D == 64)   // dense d = 128 takes the branch above
            hipLaunchKernelGGL((fa_fwd_persist_kernel<D, false>), dim3((unsigned)grid), dim3(FwdCfg<D>::THREADS), 0,
                               stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t stream) {
    return d == 64 ? launch_bf16<64>(p, stream) : launch_bf16<128>(p, stream);
}

hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t stream) {
    const unsigned nblk = (unsigned)fwd_f32_grid(p.B, p.Hq, p.N);
    if (d == 64)
        hipLaunchKernelGGL(fa_fwd_f32_kernel<64>, dim3(nblk), dim3(64), 0, stream, p);
    else
        hipLaunchKernelGGL(fa_fwd_f32_kernel<128>, dim3(nblk), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
