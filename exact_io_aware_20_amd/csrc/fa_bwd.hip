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
//   * preprocess: per query row, D = dO . O and LSE in base-2 units, written to the
//     workspace that the other two kernels read.
//   * dK/dV kernel: a workgroup owns a tile of 128 keys of one KV head (two such
//     tiles, j and ntile-1-j, under the causal rule without a window), 32 per pair of waves
//     (one forms S, P and dV, its partner dP, dS and dK one item later, P handed
//     over through LDS in bf16), streaming 64-row tiles of Q and dO of every query head in
//     the group through LDS by direct loads.  S = Q K^T is formed with the query on
//     the C rows, so P and dS feed the dV and dK contractions straight from
//     registers; the Q^T and dO^T operands of those contractions come from the same
//     natural tiles through the transposing LDS read.  The group sum over query
//     heads happens in the accumulators (no atomics, bit-reproducible).
//   * dQ kernel: a workgroup owns 32 query rows per wave of one query head (Q, dO,
//     LSE, D in registers) and streams K/V tiles like the forward; S^T = K Q^T
//     keeps each lane on one query, so LSE and D are lane-local, and the K^T
//     operand of dQ^T += K^T dS^T is read transposed from the natural K tile.
//   * Masks: tile ranges and mask tests follow the visible band as in the forward
//     (causal, full, sliding window); a block-sparse layout switches both kernels to
//     compacted lists of the tiles their blocks see (SPARSE instantiations).
#include <mutex>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// ---------------------------------------------------------------------------------
// Per query row: D_i = sum_t dO_it * O_it (fp32) and LSE_i * log2(e).  D/8 lanes
// per row, 16 bytes per lane.  A row that saw no key (LSE = -inf, possible under a
// block-sparse layout) gets +inf instead, so that its recomputed P = 2^(S - inf) is 0.
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void fa_bwd_pre_kernel(const uint16_t* o, const uint16_t* dO,
                                                              const float* lse, float* dsum, float* lse2,
                                                              float* dqacc, long long rows) {
    constexpr int LPR = D / 8;
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long row = gid / LPR;
    const int sub = (int)(gid % LPR);
    float acc = 0.f;
    if (dqacc && row < rows) {   // the fused backward's dQ accumulator starts at zero
        f32x4* z = (f32x4*)(dqacc + row * D + 8 * sub);
        z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        z[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
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
    if (row < rows && sub == 1) {
        const float l = lse[row];
        lse2[row] = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
    }
}

// ---------------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------------
template <int D>
struct DkdvCfg {
    static constexpr int WAVES = 8;          // 4 P/dV waves + 4 dS/dK waves
    static constexpr int THREADS = WAVES * kWave;
    static constexpr int BK = 4 * 32;        // keys per workgroup
    static constexpr int BQ = 64;            // query rows per streamed tile
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int NAT = SwzTile<D, 1>::ELEMS;    // natural Q or dO tile (bf16 elements)
    static constexpr int STAGE = 2 * NAT + 2 * BQ * 2;  // Q, dO, then LSE2 and D (fp32, BQ each)
    static constexpr int NSTAGE = 3;                    // items it+1 (loading), it, it-1
    static constexpr int PBUF = 2 * 4 * 32 * 64;        // bf16 P of two items: 2 x 4 pairs x 32 keys x 64 queries
    static_assert(BK == kDkdvKeys, "launch plan and kernel disagree on the key tile");
};

// Element offsets of the row fragments (row l32, chunk 2k + hh) of a MODE 1 tile;
// query half qb adds 32 qb rows, a constant.
template <int D>
struct RowOffsets {
    uint32_t off[D / 16];
    __device__ __forceinline__ void init(int l32, int hh) {
        using NT = SwzTile<D, 1>;
#pragma unroll
        for (int k = 0; k < D / 16; ++k) off[k] = (uint32_t)NT::at(l32, 2 * k + hh);
    }
};

// row fragments of the MODE 1 tile at LDS byte address `base`
template <int D>
struct RowAddr {
    uint32_t a[D / 16];
    __device__ __forceinline__ RowAddr(const RowOffsets<D>& o, uint32_t base) {
#pragma unroll
        for (int k = 0; k < D / 16; ++k) a[k] = opaque(base + 2 * o.off[k]);
    }
};

// C[q][key] = sum_d A[q][d] B[key][d] for query half qb (32 rows) of a natural
// tile and the wave's 32 keys (B fragments in registers): queries on the C rows.
template <int D>
__device__ __forceinline__ f32x16 qk_half(const RowAddr<D>& ra, const u32x4 (&bf)[D / 16], int qb) {
    f32x16 c = zero16();
#pragma unroll
    for (int k = 0; k < D / 16; ++k) c = mfma32x32x16(lds16_a(ra.a[k] + 2 * 32 * qb * D), bf[k], c);
    return c;
}

// Both query halves at once, in a scheduling region of their own: the two accumulation
// chains interleaved, and each k-step's two A fragments read AHEAD steps ahead of their
// MFMAs (a ring of AHEAD + 1 steps), so that an MFMA's operands are never the youngest
// LDS reads in flight and the wait in front of it leaves the next reads outstanding.
// The dense dK/dV reads three steps ahead; the block-sparse one measured faster at two.
template <int D, int AHEAD = 2>
__device__ __forceinline__ void qk_both(const RowAddr<D>& ra, const u32x4 (&bf)[D / 16], f32x16 (&c)[2]) {
    constexpr int K = D / 16;
    constexpr int R = AHEAD + 1;
    __builtin_amdgcn_sched_barrier(0);
    c[0] = zero16();
    c[1] = zero16();
    u32x4 a[R][2];
#pragma unroll
    for (int k = 0; k < AHEAD; ++k) {
        a[k][0] = lds16_a(ra.a[k]);
        a[k][1] = lds16_a(ra.a[k] + 2 * 32 * D);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (k + AHEAD < K) {
            a[(k + AHEAD) % R][0] = lds16_a(ra.a[k + AHEAD]);
            a[(k + AHEAD) % R][1] = lds16_a(ra.a[k + AHEAD] + 2 * 32 * D);
        }
        c[0] = mfma32x32x16(a[k % R][0], bf[k], c[0]);
        c[1] = mfma32x32x16(a[k % R][1], bf[k], c[1]);
    }
    // both chains end inside the region (a product used only later is otherwise sunk
    // past its closing fence)
    asm volatile("" : "+v"(c[0]), "+v"(c[1]));
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);   // DS reads of the first steps
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (k + AHEAD < K) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // reads of step k+AHEAD
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // MFMA, chain 0
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // MFMA, chain 1
    }
    __builtin_amdgcn_sched_barrier(0);
}

// One query half of qk_both: the chain of half qb in a scheduling region of its own,
// its A fragments read AHEAD MFMAs ahead, with the caller's independent vector work
// `vec` placed NV instructions after each MFMA.
template <int D, int AHEAD, int NV, typename F>
__device__ __forceinline__ void qk_half_mixed(const RowAddr<D>& ra, const u32x4 (&bf)[D / 16], f32x16& c, int qb,
                                              F&& vec) {
    constexpr int K = D / 16;
    constexpr int R = AHEAD + 1;
    __builtin_amdgcn_sched_barrier(0);
    vec();
    c = zero16();
    u32x4 a[R];
#pragma unroll
    for (int k = 0; k < AHEAD; ++k) a[k] = lds16_a(ra.a[k] + 2 * 32 * D * qb);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (k + AHEAD < K) a[(k + AHEAD) % R] = lds16_a(ra.a[k + AHEAD] + 2 * 32 * D * qb);
        c = mfma32x32x16(a[k % R], bf[k], c);
    }
    asm volatile("" : "+v"(c));   // the chain ends inside the region
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);   // reads of the first MFMAs
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (k + AHEAD < K) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // read of MFMA k+AHEAD
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // MFMA k
        if (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);         // vector work
    }
    __builtin_amdgcn_sched_barrier(0);
}

// acc^T += T^T X over one query half qb (2 DB MFMAs into the DB accumulators), the
// transposed A fragments read three MFMAs ahead (a ring of four), with the caller's
// independent vector work `vec` placed NV instructions after each MFMA, in one
// scheduling region.
template <int D, int NV, typename F>
__device__ __forceinline__ void acc_half_mixed(const TrAddr<D>& ta, const u32x4 (&bfh)[2], f32x16 (&acc)[D / 32],
                                               int qb, F&& vec) {
    constexpr int DB = D / 32;
    constexpr int M = 2 * DB;   // (h2, db)
    __builtin_amdgcn_sched_barrier(0);
    vec();
    u32x4 a[4];
#pragma unroll
    for (int m = 0; m < 3; ++m) a[m] = ta.frag(m % DB, 32 * qb + 16 * (m / DB));
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (m + 3 < M) a[(m + 3) & 3] = ta.frag((m + 3) % DB, 32 * qb + 16 * ((m + 3) / DB));
        acc[m % DB] = mfma32x32x16(a[m & 3], bfh[m / DB], acc[m % DB]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // transposed reads of MFMAs 0-2
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (m + 3 < M) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // reads of MFMA m+3
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA m
        if (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);     // vector work
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Set S to -inf where the query row is >= N or outside this key's band
// key - wr <= query <= key + wl, so that 2^(S*sl2 - LSE2) is exactly 0 there.
// Queries of register r: qrow0 + 8(r/4) + r%4.
__device__ __forceinline__ void mask_half(f32x16& s, int qrow0, int key, int N, int wl, int wr) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int qq = qrow0 + 8 * (r >> 2) + (r & 3);
        s[r] = (qq < N && qq >= key - wr && qq <= key + wl) ? s[r] : kNegInf;
    }
}

// Reach of the visible band (key j visible to query i iff i - wl <= j <= i + wr):
// without a window wl = N, i.e. no limit; causal means wr = 0.
__device__ __forceinline__ int band_left(const BwdParams& p) { return p.window >= 0 ? p.window : p.N; }
__device__ __forceinline__ int band_right(const BwdParams& p) {
    return p.causal ? 0 : (p.window >= 0 ? p.window : p.N);
}

// Register 4g+i of a C tile (query 8g + 4hh + i of its half) packed as k-slot
// 4(g%2)+i of B fragment g/2 (two fragments of 16 queries per half).
__device__ __forceinline__ void pack_half(const f32x16& x, u32x4 (&bf)[2]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        bf[g >> 1][2 * (g & 1)] = pack_bf16(x[4 * g], x[4 * g + 1]);
        bf[g >> 1][2 * (g & 1) + 1] = pack_bf16(x[4 * g + 2], x[4 * g + 3]);
    }
}

// acc^T += T^T X over one query half: A operand read transposed from the natural
// tile (Q or dO) that `ta` addresses, B operand the packed half `bf`.
template <int D>
__device__ __forceinline__ void acc_half(const TrAddr<D>& ta, const u32x4 (&bf)[2], f32x16 (&acc)[D / 32], int qb) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma32x32x16(ta.frag(db, 32 * qb + 16 * h2), bf[h2], acc[db]);
}

// dK/dV kernel, one 128-key tile of one KV head.  Wave w < 4 ("P/dV")
// and wave w + 4 ("dS/dK") own keys 32w .. 32w+31; the first computes S = Q K^T,
// P = 2^(S*sl2 - LSE2) and dV^T += dO^T P for item it and hands P to its partner
// through LDS, as the bf16 fragments the dV product uses; the partner, one item
// behind, computes dP = dO V^T, dS = P (dP - D) and dK^T += Q^T dS for item it-1.
// S and the exponentials are thus formed once per item.  Items are (query head of
// the group, 64-row query tile); their Q and dO tiles and LSE2/D vectors sit in
// stage it%3 of LDS, filled by direct loads, and P of item it in P slot it%2.  One
// barrier per iteration it: item it has landed and P(it-1) has been written; the
// stage of item it-2 is free and receives item it+1's loads, and P slot (it+1)%2
// was last read (P(it-1)) before this barrier.  Between barriers the P/dV wave
// runs S, mask, P, P to LDS and the dV MFMAs of item it while its partner runs P
// from LDS, dP, dS and the dK MFMAs of item it-1, so one wave of a SIMD pair runs
// exponentials or dS while the other runs matrix work.
template <int D, bool PV, bool SPARSE>
__device__ __forceinline__ void dkdv_tile(const BwdParams& p, uint16_t* smem, const uint32_t* list, int list_n,
                                          int wave, int lane, int head_kv, int kt, bool ascending) {
    using C = DkdvCfg<D>;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = p.N;
    const int G = p.Hq / p.Hkv;

    const int b = head_kv / p.Hkv;
    const int hkv = head_kv % p.Hkv;
    const int k0 = kt * C::BK;
    const int kw0 = k0 + 32 * (wave & 3);
    const int key = kw0 + l32;

    const size_t kvoff = (size_t)head_kv * N * D;
    // K (P/dV waves) or V (dS/dK waves) as B operands (lane: key, slots: 8 d)
    const uint16_t* kv = (const uint16_t*)(PV ? p.k : p.v) + kvoff;
    u32x4 bfr[C::DC];
#pragma unroll
    for (int c = 0; c < C::DC; ++c) bfr[c] = key < N ? ld_global16(kv + (size_t)key * D + 16 * c + 8 * hh) : zero_u4();
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = zero16();

    // query tiles holding a row that sees one of the workgroup's keys
    const int wl = band_left(p), wr = band_right(p);
    const int qt_start = max(0, k0 - wr) / C::BQ;
    // block-sparse: the compacted list of query tiles that see one of the workgroup's
    // two key tiles (bit 20 + j: key tile j sees it)
    const int per_head = SPARSE ? list_n : min(N - 1, k0 + C::BK - 1 + wl) / C::BQ + 1 - qt_start;
    const uint32_t wbit = 20u + (uint32_t)((wave & 3) >> 1);
    const int nitems = G * per_head;
    const float sl2 = p.scale_log2;
    // this pair's P slots (one per item parity): 64 lanes x 4 packed fragments each
    uint32_t* pbuf = (uint32_t*)(smem + C::NSTAGE * C::STAGE) + (wave & 3) * 64 * 16;

    TileDma<D, 1, C::WAVES> dma;
    dma.init(wave, lane);
    RowOffsets<D> ro;
    ro.init(l32, hh);
    TrOffsets<D> to;
    to.init(lane);
    // Items run tile-major: item it is query tile it / G (dense: from the last visible
    // tile down, or for the second tile of a pair from the first visible tile up;
    // block-sparse: list entry it / G) of query head it % G of the group.  The
    // workgroups of one KV head (its key blocks, which the launch geometry runs together
    // on one XCD) then visit the same query tiles at the same time, so that XCD's L2
    // serves their repeated reads of each Q/dO tile (most of all with many query heads
    // per KV head).
    auto item_q0 = [&](int it) {
        if constexpr (SPARSE) return (int)(list[it / G] & kSparseTileMask) * C::BQ;
        return (ascending ? qt_start + it / G : qt_start + per_head - 1 - it / G) * C::BQ;
    };
    auto issue_item = [&](int it) {
        const int hq = hkv * G + it % G;
        const int q0 = item_q0(it);
        const size_t roff = (size_t)(b * p.Hq + hq) * N + q0;
        uint16_t* st = smem + (it % C::NSTAGE) * C::STAGE;
        dma.issue((const uint16_t*)p.q + roff * D, N - q0, st, wave);
        dma.issue((const uint16_t*)p.dO + roff * D, N - q0, st + C::NAT, wave);
        // LSE2 (wave 0) and D (wave 1): 4 bytes per lane; rows >= N read row N-1
        if (wave < 2) {
            dma_row_values((wave == 0 ? p.lse2 : p.dsum) + roff, N - q0, st + 2 * C::NAT + wave * 2 * C::BQ, lane);
        }
    };
    // keys of this wave visible to some row of the item's tile
    auto active = [&](int q0) { return kw0 < N && q0 + C::BQ - 1 >= kw0 - wr && q0 <= kw0 + 31 + wl; };

    if (nitems > 0) issue_item(0);
    for (int it = 0; it <= nitems; ++it) {
        const int mine = PV ? it : it - 1;            // item this wave works on
        const bool have = PV ? it < nitems : it >= 1;
        const int q0 = have ? item_q0(mine) : 0;
        const uint16_t* st = smem + ((mine + C::NSTAGE) % C::NSTAGE) * C::STAGE;
        const float* lse2 = (const float*)(st + 2 * C::NAT);
        const float* dvec = lse2 + C::BQ;
        bool act = have && active(q0);
        if constexpr (SPARSE) act = act && ((list[have ? mine / G : 0] >> wbit) & 1u);   // no read past the list
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();                                               // A
        if (it + 1 < nitems) issue_item(it + 1);
        // Each wave overlaps its own vector work with its own matrix work: the second
        // query half's vector work runs in the scheduling region of the first half's
        // dV or dK products (P/dV: exponentials, bf16 packing and the hand-over of P;
        // dS/dK: unpacking the handed-over P, dS = P (dP - D) and its packing).
        f32x16 x[2];                                                   // P (P/dV) or dP (dS/dK)
        u32x4 bf[2][2];                                                // P or dS, bf16 B fragments
        // the wave whose result the other waits on issues first: P/dV while it forms
        // P, dS/dK while it forms dS and dK
        __builtin_amdgcn_s_setprio(PV ? 2 : 0);
        if (act) {
            if constexpr (PV) {
                const bool mask = q0 < kw0 + 31 - wr || q0 + C::BQ > N || q0 + C::BQ - 1 > kw0 + wl;
                uint32_t* pb = pbuf + (mine & 1) * 4 * 64 * 16;
                f32x4 L[2][4];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) L[qb][g] = *(const f32x4*)(lse2 + 32 * qb + 8 * g + 4 * hh);
                // P of one half: 2^(S sl2 - LSE2), packed to bf16 and handed over
                auto probs = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            x[qb][4 * g + i] = fast_exp2(__builtin_fmaf(x[qb][4 * g + i], sl2, -L[qb][g][i]));
                    pack_half(x[qb], bf[qb]);
                };
                auto hand_over = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) *(u32x4*)(pb + ((2 * qb + h2) * 64 + lane) * 4) = bf[qb][h2];
                };
                const RowAddr<D> ra(ro, lds_addr(st));
                if (!mask) {
                    // S one query half at a time: half 0's exponentials run under half 1's
                    // products (the empty asm pins their start inside that region)
                    qk_half_mixed<D, SPARSE ? 2 : 3, 0>(ra, bfr, x[0], 0, [] {});
                    qk_half_mixed<D, SPARSE ? 2 : 3, 3>(ra, bfr, x[1], 1, [&] {
                        asm volatile("" : "+v"(x[0]));
                        probs(0);
                    });
                } else {
                    qk_both<D, SPARSE ? 2 : 3>(ra, bfr, x);
                    if (mask) {
#pragma unroll
                        for (int qb = 0; qb < 2; ++qb) mask_half(x[qb], q0 + 32 * qb + 4 * hh, key, N, wl, wr);
                    }
                    probs(0);
                }
                hand_over(0);
                __builtin_amdgcn_s_setprio(0);
                const TrAddr<D> ta(to, lds_addr(st + C::NAT));
                // The empty asm pins the start of half 1's vector work inside the region (pure
                // arithmetic is otherwise free to be placed before it).  Its hand-over is
                // written after the region: the compiler cannot tell that store from the
                // region's dO reads apart, and would order every read behind it.
                acc_half_mixed<D, 3>(ta, bf[0], acc, 0, [&] {                 // dV^T += dO^T P, half 0
                    asm volatile("" : "+v"(x[1]));
                    probs(1);
                });
                hand_over(1);
                acc_half_mixed<D, 0>(ta, bf[1], acc, 1, [] {});               // half 1
            } else {
                const uint32_t* pb = pbuf + (mine & 1) * 4 * 64 * 16;
                u32x4 praw[2][2];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) praw[qb][h2] = *(const u32x4*)(pb + ((2 * qb + h2) * 64 + lane) * 4);
                f32x4 Dd[2][4];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) Dd[qb][g] = *(const f32x4*)(dvec + 32 * qb + 8 * g + 4 * hh);
                // dS = P (dP - D), P unpacked from the hand-over as it is used: register
                // 4g+i of a half is the low (i even) or high bf16 of word 2(g%2) + i/2 of
                // fragment g/2 (the inverse of pack_half)
                auto dsoft = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t w = praw[qb][g >> 1][2 * (g & 1) + (i >> 1)];
                            const float pv = (i & 1) ? bf16_hi(w) : bf16_lo(w);
                            x[qb][4 * g + i] = pv * (x[qb][4 * g + i] - Dd[qb][g][i]);
                        }
                    pack_half(x[qb], bf[qb]);
                };
                const RowAddr<D> ra(ro, lds_addr(st + C::NAT));
                // dP = dO V^T one query half at a time, half 0's dS under half 1's products
                qk_half_mixed<D, SPARSE ? 2 : 3, 0>(ra, bfr, x[0], 0, [] {});
                __builtin_amdgcn_s_setprio(2);
                qk_half_mixed<D, SPARSE ? 2 : 3, 4>(ra, bfr, x[1], 1, [&] {
                    asm volatile("" : "+v"(x[0]));
                    dsoft(0);
                });
                const TrAddr<D> ta(to, lds_addr(st));
                acc_half_mixed<D, 4>(ta, bf[0], acc, 0, [&] {                 // dK^T += Q^T dS, half 0
                    asm volatile("" : "+v"(x[1]));
                    dsoft(1);
                });
                acc_half_mixed<D, 0>(ta, bf[1], acc, 1, [] {});               // half 1
            }
        } else {
            __builtin_amdgcn_s_setprio(PV ? 0 : 2);
        }
    }

    __builtin_amdgcn_s_setprio(0);
    if (key < N) {
        uint16_t* dst = (uint16_t*)(PV ? p.dv : p.dk) + kvoff + (size_t)key * D;
        const float sc = PV ? 1.f : p.scale;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(u32x2*)(dst + 32 * db + 8 * g + 4 * hh) =
                    u32x2{pack_bf16(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc),
                          pack_bf16(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc)};
    }
}

// A workgroup's key tiles.  Causal without a window: a pair, tile j walked from its
// last visible query tile down, then tile ntile_k - 1 - j walked from its first visible
// query tile up.  Every pair then holds the same number of items, so the workgroups end
// together, and all workgroups of a KV head read the same query tile at the same time in
// both halves (the first halves all start at the last tile; a second half starts where
// its first ended, at a time that puts it on the same tile as every other second half).
// Full attention, a window or a block-sparse layout: one tile, walked down; there the
// tiles' lengths already match (up to the window's ends) and pairing only halves the grid.
template <int D, bool PV, bool SPARSE>
__device__ __forceinline__ void dkdv_role(const BwdParams& p, uint16_t* smem, const uint32_t* list, int list_n,
                                          int wave, int lane) {
    using C = DkdvCfg<D>;
    const int ntile_k = (p.N + C::BK - 1) / C::BK;
    const bool paired = !SPARSE && p.causal && p.window < 0;
    int head_kv, kt;
    // Paired workgroups all hold the same work, and so do a window's tiles (one band
    // each): the workgroups of one head, side by side on one XCD, then stream that head's
    // Q/dO tiles through its L2 together.  Causal tiles without a pair differ in length,
    // and there groups of four heads measured faster.
    map_block(blockIdx.x, gridDim.x, paired ? (ntile_k + 1) / 2 : ntile_k, p.B * p.Hkv, false, head_kv, kt,
              (paired || p.window >= 0) ? 1 : 4);
    dkdv_tile<D, PV, SPARSE>(p, smem, list, list_n, wave, lane, head_kv, kt, false);
    const int kt2 = ntile_k - 1 - kt;
    if (paired && kt2 != kt) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();   // every wave done with the first tile's LDS stages and P slots
        dkdv_tile<D, PV, SPARSE>(p, smem, list, list_n, wave, lane, head_kv, kt2, true);
    }
}

template <int D, bool SPARSE>
__global__ __launch_bounds__(DkdvCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(BwdParams p) {
    using C = DkdvCfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::NSTAGE * C::STAGE + C::PBUF];
    __shared__ uint32_t list[SPARSE ? kSparseMaxBlocks : 1];
    __shared__ int list_n;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave < C::WAVES);
    int n = 0;
    if constexpr (SPARSE) {
        // query tiles u that see key tile kt0 + j of this workgroup (layout bit set,
        // and not before the key tile under the causal rule)
        const int N = p.N;
        const int nb = (N + kSparseBlock - 1) / kSparseBlock;
        const int ntile_k = (N + C::BK - 1) / C::BK;
        int head_kv, kt;
        map_block(blockIdx.x, gridDim.x, ntile_k, p.B * p.Hkv, false, head_kv, kt, 4);
        const int kt0 = kt * (C::BK / kSparseBlock);
        if (wave == 0) {
            // The layout is read down a column here (one row per lane), so batching the
            // reads gained nothing when measured: one group at a time, each read only
            // where the causal rule leaves the pair.
            const int u_begin = p.causal ? min(kt0, nb) : 0;   // earlier query tiles are masked
            const int c = compact_tiles<1>(list, u_begin, nb, tid & 63, [&](int u) -> uint32_t {
                uint32_t bits = 0;
#pragma unroll
                for (int j = 0; j < C::BK / kSparseBlock; ++j) {
                    const int kb = kt0 + j;
                    if (kb < nb && (!p.causal || u >= kb) && p.block_mask[(size_t)u * nb + kb]) bits |= 1u << j;
                }
                return bits;
            });
            if ((tid & 63) == 0) list_n = c;
        }
        __syncthreads();
        n = list_n;
    }
    if (wave < 4)
        dkdv_role<D, true, SPARSE>(p, smem, list, n, wave, tid & 63);
    else
        dkdv_role<D, false, SPARSE>(p, smem, list, n, wave, tid & 63);
}


// ---------------------------------------------------------------------------------
// Fused dK/dV/dQ kernel.  A workgroup owns 128 keys of one KV head, as the dK/dV
// kernel above, and also forms dQ = scale dS K for every item it visits: the dS tile
// of the item (64 queries x 128 keys, bf16) goes to LDS, and every query row's dQ
// contribution is added in fp32 to an accumulator in the workspace with vector
// atomics (global_atomic_add_f32); a convert kernel scales it into bf16 dQ once all
// key blocks are done.  So S and dP are formed once per (query, key) pair for all
// three gradients: five contractions instead of the seven of the dK/dV + dQ pair.
//
// Roles: wave w < 4 (P/dV) and w + 4 (dS/dK) share a SIMD and own keys 32w..32w+31,
// as before, but both now work on the same item, with two barriers per item:
//   A  item it has landed (stage it & 1); the dS of item it-1 is complete.
//   phase 1: P/dV forms S, P and writes P (bf16 fragments) to slot it & 1;
//            dS/dK forms dQ of item it-1 (one 32 x 32 tile), then dP = dO V^T.
//   B  P(it) is visible.
//   phase 2: P/dV forms dV^T += dO^T P, then its dQ tile of item it-1;
//            dS/dK reads P, forms dS = P (dP - D), writes dS over P in natural
//            [key][query] layout, and dK^T += Q^T dS.
// The dQ tile products read dS transposed (A operand: query rows, keys along k) and
// the workgroup's K tile transposed (B operand: d columns, keys along k), both with
// the transposing LDS read.  Two Q/dO stages, K (two 64-key tiles) and two P/dS slots
// fit the LDS (129 KB at d = 128).  Items run tile-major (query tiles from last to
// first, the group's query heads within a tile), as in the dK/dV kernel.
// Keys at or beyond N are masked like hidden pairs (P = 0, so dS = 0).
// ---------------------------------------------------------------------------------
template <int D>
struct FusedCfg {
    static constexpr int WAVES = 8;
    static constexpr int THREADS = WAVES * kWave;
    static constexpr int BK = 128;                        // keys per workgroup
    static constexpr int BQ = 64;                         // query rows per item
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int NAT = SwzTile<D, 1>::ELEMS;      // one 64-row Q, dO or K tile (bf16 elements)
    static constexpr int STAGE = 2 * NAT + 2 * BQ * 2;    // Q, dO, then LSE2 and D (fp32, BQ each)
    static constexpr int KOFF = 2 * STAGE;                // K of the workgroup: two 64-key tiles
    static constexpr int SOFF = KOFF + 2 * NAT;           // two P / dS slots
    static constexpr int SLOT = BK * BQ;                  // bf16 elements of one slot
    static constexpr int TOTAL = SOFF + 2 * SLOT;
    static_assert(BK == kDkdvKeys, "launch plan and kernel disagree on the key tile");
    static_assert(TOTAL * 2 <= 160 * 1024, "LDS budget");
};

// S for query half qb of an item: -inf where the query row is >= N, the key is >= N,
// or the pair is outside the band (so that 2^(S*sl2 - LSE2) is exactly 0 there).
__device__ __forceinline__ void fused_mask_half(f32x16& s, int qrow0, int key, int N, int wl, int wr) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int qq = qrow0 + 8 * (r >> 2) + (r & 3);
        s[r] = (key < N && qq < N && qq >= key - wr && qq <= key + wl) ? s[r] : kNegInf;
    }
}

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8) that waits for every LDS operation and for all but the n youngest vector
// memory operations of the wave (they retire in issue order).
constexpr int wait_lgkm0_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
constexpr int kDqAtomics = 16;   // atomic adds of one dQ tile (one per C register)

// Workgroup barrier of the fused kernel.  Each wave first waits for its LDS writes and
// for its direct loads of the next item, but not for the dQ atomics it issued after
// those loads (`pending` of them): __syncthreads() would wait for those too (its fence
// covers global memory), and the atomics, which nothing in the workgroup reads, would
// then stall every item.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void fused_barrier(bool pending) {
    asm volatile("" ::: "memory");
    if (pending)
        __builtin_amdgcn_s_waitcnt(wait_lgkm0_vm(kDqAtomics));
    else
        __builtin_amdgcn_s_waitcnt(wait_lgkm0_vm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Mid-item barrier: only LDS writes (the P of the item) must be complete; the next
// item's direct loads and the dQ atomics stay in flight.
__device__ __forceinline__ void fused_lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wait_lgkm0_vm(63));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int D, bool PV>
__device__ __forceinline__ void fused_role(const BwdParams& p, uint16_t* smem, int wave, int lane) {
    using C = FusedCfg<D>;
    using DS = SwzTile<64, 1>;   // dS tile: 64 key rows x 64 query columns
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = p.N;
    const int G = p.Hq / p.Hkv;

    const int ntile_k = (N + C::BK - 1) / C::BK;
    int head_kv, kt;
    map_block(blockIdx.x, gridDim.x, ntile_k, p.B * p.Hkv, false, head_kv, kt, 4);
    const int b = head_kv / p.Hkv;
    const int hkv = head_kv % p.Hkv;
    const int k0 = kt * C::BK;
    const int pair = wave & 3;
    const int kw0 = k0 + 32 * pair;
    const int key = kw0 + l32;

    const size_t kvoff = (size_t)head_kv * N * D;
    // K (P/dV waves) or V (dS/dK waves) as B operands (lane: key, slots: 8 d)
    const uint16_t* kv = (const uint16_t*)(PV ? p.k : p.v) + kvoff;
    u32x4 bfr[C::DC];
#pragma unroll
    for (int c = 0; c < C::DC; ++c) bfr[c] = key < N ? ld_global16(kv + (size_t)key * D + 16 * c + 8 * hh) : zero_u4();
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = zero16();

    const int wl = band_left(p), wr = band_right(p);
    const int qt_start = max(0, k0 - wr) / C::BQ;
    const int per_head = min(N - 1, k0 + C::BK - 1 + wl) / C::BQ + 1 - qt_start;
    const int nitems = G * per_head;
    const float sl2 = p.scale_log2;

    // this wave's dQ tile of an item: queries 32 qh .. +31, d columns 32 dbq .. +31
    // (d = 128: every wave one of the eight; d = 64: the four P/dV waves)
    constexpr bool kAllWaves = D == 128;
    const bool dq_wave = kAllWaves || PV;
    const int qh = kAllWaves ? (wave >> 2) : (pair >> 1);
    const int dbq = kAllWaves ? (wave & 3) : (pair & 1);

    uint16_t* ktile = smem + C::KOFF;
    uint16_t* slots = smem + C::SOFF;

    TileDma<D, 1, C::WAVES> dma;
    dma.init(wave, lane);
    RowOffsets<D> ro;
    ro.init(l32, hh);
    TrOffsets<D> to;
    to.init(lane);
    TrColOffsets<64> dso;    // dS tile, query block qh
    dso.init(lane, qh);
    TrColOffsets<D> kco;     // K tile, d block dbq
    kco.init(lane, dbq);

    auto item_q0 = [&](int it) { return (qt_start + per_head - 1 - it / G) * C::BQ; };
    auto item_row = [&](int it) { return (size_t)(b * p.Hq + hkv * G + it % G) * N + item_q0(it); };
    auto issue_item = [&](int it) {
        const int q0 = item_q0(it);
        const size_t roff = item_row(it);
        uint16_t* st = smem + (it & 1) * C::STAGE;
        dma.issue((const uint16_t*)p.q + roff * D, N - q0, st, wave);
        dma.issue((const uint16_t*)p.dO + roff * D, N - q0, st + C::NAT, wave);
        // LSE2 (wave 0) and D (wave 1): 4 bytes per lane; rows >= N read row N-1
        if (wave < 2) {
            dma_row_values((wave == 0 ? p.lse2 : p.dsum) + roff, N - q0, st + 2 * C::NAT + wave * 2 * C::BQ, lane);
        }
    };
    auto active = [&](int q0) { return kw0 < N && q0 + C::BQ - 1 >= kw0 - wr && q0 <= kw0 + 31 + wl; };

    // dQ tile of item j from its dS (slot j & 1) and the workgroup's K, added to the
    // fp32 accumulator by exactly kDqAtomics atomic instructions (fused_barrier counts
    // them): a row >= N has dS = 0, so its exact zero is added to row N-1 instead
    auto dq_products = [&](int j) {
        const uint16_t* dsl = slots + (j & 1) * C::SLOT;
        f32x16 c = zero16();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const TrColAddr<64> sa(dso, lds_addr(dsl + t * DS::ELEMS));
            const TrColAddr<D> ka(kco, lds_addr(ktile + t * C::NAT));
#pragma unroll
            for (int kk = 0; kk < 64; kk += 16) c = mfma32x32x16(sa.frag(kk), ka.frag(kk), c);
        }
        const int q0 = item_q0(j);
        const int qbase = q0 + 32 * qh + 4 * hh;
        float* dst = p.dqacc + (item_row(j) - q0) * D + 32 * dbq + l32;   // row 0 of the head
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qq = min(qbase + 8 * (r >> 2) + (r & 3), N - 1);
            atomicAddNoRet(dst + (size_t)qq * D, c[r]);
        }
    };

    if (nitems > 0) {
        // the workgroup's K (both 64-key tiles; a tile past N reads row N-1, finite, and
        // its dS is 0) with the first item
        const uint16_t* kh = (const uint16_t*)p.k + kvoff;
        dma.issue(kh + (size_t)k0 * D, N - k0, ktile, wave);
        const int k1 = min(k0 + 64, N - 1);
        dma.issue(kh + (size_t)k1 * D, max(1, N - (k0 + 64)), ktile + C::NAT, wave);
        issue_item(0);
    }
    u32x4 bf[2][2];   // P/dV: P of the item (B fragments of dV), kept across the mid barrier
    f32x16 x[2];      // dS/dK: dP of the item, kept across the mid barrier
    for (int it = 0; it <= nitems; ++it) {
        const bool have = it < nitems;
        const int q0 = have ? item_q0(it) : 0;
        const uint16_t* st = smem + (it & 1) * C::STAGE;
        const float* lse2 = (const float*)(st + 2 * C::NAT);
        const float* dvec = lse2 + C::BQ;
        const bool act = have && active(q0);
        uint32_t* pslot = (uint32_t*)(slots + (it & 1) * C::SLOT) + pair * 64 * 16;
        // A: item it has landed (the dQ atomics of the previous iteration may still be in
        // flight), dS(it-1) is written
        fused_barrier(dq_wave && it >= 2);
        if (it + 1 < nitems) issue_item(it + 1);
        // ---- phase 1
        if constexpr (PV) {
            __builtin_amdgcn_s_setprio(2);
            if (act) {
                const bool mask = q0 < kw0 + 31 - wr || q0 + C::BQ > N || q0 + C::BQ - 1 > kw0 + wl || kw0 + 31 >= N;
                {
                    const RowAddr<D> ra(ro, lds_addr(st));
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) x[qb] = qk_half<D>(ra, bfr, qb);
                }
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    if (mask) fused_mask_half(x[qb], q0 + 32 * qb + 4 * hh, key, N, wl, wr);
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 L = *(const f32x4*)(lse2 + 32 * qb + 8 * g + 4 * hh);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            x[qb][4 * g + i] = fast_exp2(__builtin_fmaf(x[qb][4 * g + i], sl2, -L[i]));
                    }
                    pack_half(x[qb], bf[qb]);
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) *(u32x4*)(pslot + ((2 * qb + h2) * 64 + lane) * 4) = bf[qb][h2];
                }
            }
            __builtin_amdgcn_s_setprio(0);
        } else {
            if (it > 0 && dq_wave) dq_products(it - 1);
            if (act) {
                const RowAddr<D> ra(ro, lds_addr(st + C::NAT));
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) x[qb] = qk_half<D>(ra, bfr, qb);
            }
        }
        fused_lds_barrier();                                           // B: P(it) is written
        // ---- phase 2
        if constexpr (PV) {
            if (act) {
                const TrAddr<D> ta(to, lds_addr(st + C::NAT));
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) acc_half<D>(ta, bf[qb], acc, qb);   // dV^T += dO^T P
            }
            if (it > 0 && dq_wave) dq_products(it - 1);
        } else {
            uint16_t* dsrow = slots + (it & 1) * C::SLOT + (pair >> 1) * DS::ELEMS;
            const int r = 32 * (pair & 1) + l32;   // this lane's key row in its 64-key dS tile
            if (act) {
                __builtin_amdgcn_s_setprio(2);
                f32x16 pp[2];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const u32x4 v = *(const u32x4*)(pslot + ((2 * qb + h2) * 64 + lane) * 4);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            // inverse of pack_half: word j of fragment h2 holds registers
                            // r and r + 1, r = 4 (2 h2 + j/2) + 2 (j%2)
                            const int rr = 4 * (2 * h2 + (j >> 1)) + 2 * (j & 1);
                            pp[qb][rr] = bf16_lo(v[j]);
                            pp[qb][rr + 1] = bf16_hi(v[j]);
                        }
                    }
                u32x4 dsf[2][2];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 Dd = *(const f32x4*)(dvec + 32 * qb + 8 * g + 4 * hh);
                        float v[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) v[i] = pp[qb][4 * g + i] * (x[qb][4 * g + i] - Dd[i]);
                        // registers 4g..4g+3: queries 32 qb + 8 g + 4 hh + 0..3; packed as
                        // pack_half packs them (B fragment g/2, words 2(g%2), 2(g%2)+1), and
                        // written to the natural [key][query] dS tile in one 8-byte store
                        const uint32_t lo = pack_bf16(v[0], v[1]), hi = pack_bf16(v[2], v[3]);
                        if (g == 0) { dsf[qb][0][0] = lo; dsf[qb][0][1] = hi; }
                        if (g == 1) { dsf[qb][0][2] = lo; dsf[qb][0][3] = hi; }
                        if (g == 2) { dsf[qb][1][0] = lo; dsf[qb][1][1] = hi; }
                        if (g == 3) { dsf[qb][1][2] = lo; dsf[qb][1][3] = hi; }
                        *(u32x2*)(dsrow + DS::at(r, 4 * qb + g) + 4 * hh) = u32x2{lo, hi};
                    }
                }
                __builtin_amdgcn_s_setprio(0);
                const TrAddr<D> ta(to, lds_addr(st));
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) acc_half<D>(ta, dsf[qb], acc, qb);   // dK^T += Q^T dS
            } else if (have) {
                // no key of this pair sees the item: its dS rows are zero
#pragma unroll
                for (int c = 0; c < 8; ++c) *(u32x2*)(dsrow + DS::at(r, c) + 4 * hh) = u32x2{0u, 0u};
            }
        }
    }

    if (key < N) {
        uint16_t* dst = (uint16_t*)(PV ? p.dv : p.dk) + kvoff + (size_t)key * D;
        const float sc = PV ? 1.f : p.scale;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(u32x2*)(dst + 32 * db + 8 * g + 4 * hh) =
                    u32x2{pack_bf16(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc),
                          pack_bf16(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc)};
    }
}

template <int D>
__global__ __launch_bounds__(FusedCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_fused_kernel(BwdParams p) {
    using C = FusedCfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::TOTAL];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave < C::WAVES);
    if (wave < 4)
        fused_role<D, true>(p, smem, wave, tid & 63);
    else
        fused_role<D, false>(p, smem, wave, tid & 63);
}

// dQ = scale * accumulator, rounded to bf16 (round to nearest even): 8 values per lane.
template <int D>
__global__ __launch_bounds__(kThreads) void fa_bwd_dq_convert_kernel(const float* dqacc, uint16_t* dq, float scale,
                                                                     long long n8) {
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n8) return;
    const f32x4 a = *(const f32x4*)(dqacc + 8 * i);
    const f32x4 c = *(const f32x4*)(dqacc + 8 * i + 4);
    *(u32x4*)(dq + 8 * i) = u32x4{pack_bf16(a[0] * scale, a[1] * scale), pack_bf16(a[2] * scale, a[3] * scale),
                                  pack_bf16(c[0] * scale, c[1] * scale), pack_bf16(c[2] * scale, c[3] * scale)};
}

// ---------------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------------
template <int D>
struct DqCfg {
    static constexpr int WAVES = 8;
    static constexpr int THREADS = WAVES * kWave;
    static constexpr int BR = WAVES * 32;
    static constexpr int BC = 64;
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int KT = SwzTile<D, 1>::ELEMS;   // K: fragment and transposing reads
    static constexpr int VT = SwzTile<D, 0>::ELEMS;   // V: fragment reads
    static constexpr int STAGE = KT + VT;
    static_assert(BR == kDqRows, "launch plan and kernel disagree on the row tile");
};

// S^T = K Q^T and dP^T = V dO^T of one key tile in a scheduling region of their own:
// the four accumulation chains (S and dP of the two 32-key blocks) taken in turn, chunk
// by chunk, each A fragment read two MFMAs ahead (a ring of three), so that a read is
// never waited for by the MFMA right behind it.  Every register accumulates its chunks
// in the same order as a plain loop over them.
template <int D>
__device__ __forceinline__ void dq_scores(const uint16_t* st, const u32x4 (&qf)[D / 16], const u32x4 (&gf)[D / 16],
                                          f32x16 (&s)[2], f32x16 (&dp)[2], int l32, int hh) {
    using C = DqCfg<D>;
    using KS = SwzTile<D, 1>;
    using VS = SwzTile<D, 0>;
    constexpr int M = 4 * C::DC;   // m: chunk m/4, r = m%4: S block 0, dP block 0, S block 1, dP block 1
    auto frag = [&](int m) __attribute__((always_inline)) -> u32x4 {
        const int c = m >> 2, r = m & 3, kb = r >> 1;
        if ((r & 1) == 0) return lds16(st + KS::at(32 * kb + l32, 2 * c + hh));
        return lds16(st + C::KT + VS::at(32 * kb + l32, 2 * c + hh));
    };
    __builtin_amdgcn_sched_barrier(0);
    s[0] = zero16();
    s[1] = zero16();
    dp[0] = zero16();
    dp[1] = zero16();
    u32x4 a[3];
    a[0] = frag(0);
    a[1] = frag(1);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (m + 2 < M) a[(m + 2) % 3] = frag(m + 2);
        const int c = m >> 2, r = m & 3, kb = r >> 1;
        if ((r & 1) == 0)
            s[kb] = mfma32x32x16(a[m % 3], qf[c], s[kb]);
        else
            dp[kb] = mfma32x32x16(a[m % 3], gf[c], dp[kb]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // reads of MFMAs 0 and 1
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (m + 2 < M) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // read of MFMA m+2
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA m
    }
    __builtin_amdgcn_sched_barrier(0);
}

// dQ kernel: per key/value tile, S^T = K Q^T and dP^T = V dO^T (lane: query),
// dS^T = P^T (dP^T - D) rounded to bf16, dQ^T += K^T dS^T with K^T read transposed
// from the natural K tile.  K/V tiles are double-buffered with one barrier each.
template <int D, bool SPARSE>
__global__ __launch_bounds__(DqCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(BwdParams p) {
    using C = DqCfg<D>;
    using KS = SwzTile<D, 1>;
    using VS = SwzTile<D, 0>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];
    __shared__ uint32_t list[SPARSE ? kSparseMaxBlocks : 1];
    __shared__ int list_n;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave < C::WAVES);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int N = p.N;

    const int ntile_q = (N + C::BR - 1) / C::BR;
    int head, qt;
    map_block(blockIdx.x, gridDim.x, ntile_q, p.B * p.Hq, p.causal != 0, head, qt, 4);
    const int hq = head % p.Hq;
    const int b = head / p.Hq;
    const int hkv = hq / (p.Hq / p.Hkv);
    const size_t qoff = (size_t)head * N * D;
    const size_t kvoff = ((size_t)b * p.Hkv + hkv) * N * D;
    const uint16_t* Kh = (const uint16_t*)p.k + kvoff;
    const uint16_t* Vh = (const uint16_t*)p.v + kvoff;

    const int q0 = qt * C::BR;
    const int qw0 = q0 + wave * 32;
    const int q = qw0 + l32;
    const int q_last = min(q0 + C::BR, N) - 1;
    // tiles [t_begin, ntiles) hold a key visible to some row of the workgroup
    const int wl = band_left(p), wr = band_right(p);
    const int t_begin = max(0, q0 - wl) / C::BC;
    const int ntiles = min(N - 1, q_last + wr) / C::BC + 1;
    const int wq_last = min(qw0 + 32, N) - 1;
    const int wave_tiles = wq_last < qw0 ? 0 : min(N - 1, wq_last + wr) / C::BC + 1;

    // Q and dO as B operands of S^T = K Q^T and dP^T = V dO^T (lane: query)
    u32x4 qf[C::DC], gf[C::DC];
    const bool ok = q < N;
#pragma unroll
    for (int c = 0; c < C::DC; ++c) {
        qf[c] = ok ? ld_global16((const uint16_t*)p.q + qoff + (size_t)q * D + 16 * c + 8 * hh) : zero_u4();
        gf[c] = ok ? ld_global16((const uint16_t*)p.dO + qoff + (size_t)q * D + 16 * c + 8 * hh) : zero_u4();
    }
    float lse2, dd;
    if (p.form_rows) {
        // The per-row terms formed here, bit for bit as fa_bwd_pre_kernel forms them:
        // D = dO . O as one fma chain per 8-element chunk j = 2c + hh, the chunks then
        // summed pairwise over j ^ D/16, ..., j ^ 2 (in this lane) and j ^ 1 (the other
        // half of the row, lane ^ 32); LSE in base 2, +inf for a row that saw no key.
        // Written to the workspace for the dK/dV kernel.
        float part[C::DC];
#pragma unroll
        for (int c = 0; c < C::DC; ++c) {
            const u32x4 a = ok ? ld_global16((const uint16_t*)p.o + qoff + (size_t)q * D + 16 * c + 8 * hh) : zero_u4();
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc = __builtin_fmaf(bf16_lo(a[w]), bf16_lo(gf[c][w]), acc);
                acc = __builtin_fmaf(bf16_hi(a[w]), bf16_hi(gf[c][w]), acc);
            }
            part[c] = acc;
        }
#pragma unroll
        for (int m = C::DC / 2; m >= 1; m >>= 1)
#pragma unroll
            for (int c = 0; c < m; ++c) part[c] = part[c] + part[c + m];
        dd = part[0] + __shfl_xor(part[0], 32);
        const float l = ok ? p.lse[(size_t)head * N + q] : 0.f;
        lse2 = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
        if (ok && hh == 0) {
            p.dsum[(size_t)head * N + q] = dd;
            p.lse2[(size_t)head * N + q] = lse2;
        }
    } else {
        lse2 = ok ? p.lse2[(size_t)head * N + q] : 0.f;
        dd = ok ? p.dsum[(size_t)head * N + q] : 0.f;
    }
    f32x16 dqt[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) dqt[db] = zero16();
    const float sl2 = p.scale_log2;

    TileDma<D, 1, C::WAVES> kdma;
    TileDma<D, 0, C::WAVES> vdma;
    kdma.init(wave, lane);
    vdma.init(wave, lane);
    auto load_tile = [&](int t, uint16_t* st) {
        const int k0 = t * C::BC;
        kdma.issue(Kh + (size_t)k0 * D, N - k0, st, wave);
        vdma.issue(Vh + (size_t)k0 * D, N - k0, st + C::KT, wave);
    };

    // Entries e in [e_begin, e_end): the key tiles t_begin .. ntiles-1, or under a
    // block-sparse layout the compacted list of key tiles that one of the workgroup's
    // four 64-row blocks sees (bit 20 + j: block j sees it).
    int e_begin = t_begin, e_end = ntiles;
    if constexpr (SPARSE) {
        const int nb = (N + kSparseBlock - 1) / kSparseBlock;
        const int qb0 = q0 / kSparseBlock;
        if (wave == 0) {
            const int u_end = p.causal ? min(nb, qb0 + C::BR / kSparseBlock) : nb;   // later key tiles are masked
            const int c = compact_tiles(list, 0, u_end, lane, [&](int u) -> uint32_t {
                uint32_t bits = 0;
#pragma unroll
                for (int j = 0; j < C::BR / kSparseBlock; ++j) {
                    const int qb = qb0 + j;
                    const bool set = p.block_mask[(size_t)min(qb, nb - 1) * nb + u] != 0;
                    bits |= (uint32_t)((qb < nb) & (!p.causal | (u <= qb)) & set) << j;
                }
                return bits;
            });
            if (lane == 0) list_n = c;
        }
        __syncthreads();
        e_begin = 0;
        e_end = list_n;
    }
    const uint32_t wbit = 20u + (uint32_t)(wave / (kSparseBlock / 32));
    auto tile_of = [&](int e) { return SPARSE ? (int)(list[e] & kSparseTileMask) : e; };

    if (e_begin < e_end) load_tile(tile_of(e_begin), smem + (e_begin & 1) * C::STAGE);
    for (int e = e_begin; e < e_end; ++e) {
        const int t = tile_of(e);
        const int k0 = t * C::BC;
        const uint16_t* st = smem + (e & 1) * C::STAGE;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();                       // tile e landed; stage (e+1)&1 free
        if (e + 1 < e_end) load_tile(tile_of(e + 1), smem + ((e + 1) & 1) * C::STAGE);

        if (t < wave_tiles && (!SPARSE || ((list[e] >> wbit) & 1u))) {
            // S and dP products at raised issue priority, so that a wave in this block
            // keeps the matrix pipe fed while its SIMD partner runs dS (measured
            // 0.4-0.5 % faster than equal priorities)
            __builtin_amdgcn_s_setprio(3);
            f32x16 s[2], dp[2];
            dq_scores<D>(st, qf, gf, s, dp, l32, hh);
            if (k0 + C::BC - 1 > qw0 + wr || k0 + C::BC > N || k0 < wq_last - wl) {
                const int lo = q - wl, hi = min(q + wr, N - 1);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                        const bool vis = kk >= lo && kk <= hi;
                        s[kb][r] = vis ? s[kb][r] : kNegInf;   // -inf * sl2 - lse2 -> p = 0
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
            u32x4 dsf[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 8 * h2 + 2 * j;
                        const float pa = fast_exp2(__builtin_fmaf(s[kb][r], sl2, -lse2));
                        const float pb = fast_exp2(__builtin_fmaf(s[kb][r + 1], sl2, -lse2));
                        dsf[kb][h2][j] = pack_bf16(pa * (dp[kb][r] - dd), pb * (dp[kb][r + 1] - dd));
                    }
            // ---- dQ^T += K^T dS^T  (contraction over the keys)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
                        dqt[db] = mfma32x32x16(tr_frag<D>(st, db, 32 * kb + 16 * h2, lane), dsf[kb][h2], dqt[db]);
        }
    }

    if (ok) {
        uint16_t* dQh = (uint16_t*)p.dq + qoff + (size_t)q * D;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(u32x2*)(dQh + 32 * db + 8 * g + 4 * hh) =
                    u32x2{pack_bf16(dqt[db][4 * g] * sc, dqt[db][4 * g + 1] * sc),
                          pack_bf16(dqt[db][4 * g + 2] * sc, dqt[db][4 * g + 3] * sc)};
    }
}

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------
// ---------------------------------------------------------------------------------
// Static scratch of the no-allocation backward: 2 x kScratchRows fp32 (D, then LSE in
// base 2), 16 MiB held on every device the library runs on until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory): its device address is looked up once per device,
// with that device current, and kept.
// ---------------------------------------------------------------------------------
static __device__ __align__(256) float scratch[2 * kScratchRows];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t bwd_scratch(hipStream_t stream, float** ptr) {
    int dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = (float*)p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

template <int D>
static hipError_t launch_pre(const BwdParams& p, hipStream_t stream) {
    const long long rows = (long long)p.B * p.Hq * p.N;
    const unsigned blocks = (unsigned)((rows * (D / 8) + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(fa_bwd_pre_kernel<D>, dim3(blocks), dim3(kThreads), 0, stream,
                       (const uint16_t*)p.o, (const uint16_t*)p.dO, p.lse, p.dsum, p.lse2, p.dqacc, rows);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv(const BwdParams& p, hipStream_t stream) {
    // one workgroup per pair of key tiles (causal, no window) or per key tile
    const long long ntk = (p.N + DkdvCfg<D>::BK - 1) / DkdvCfg<D>::BK;
    const bool paired = !p.block_mask && p.causal && p.window < 0;
    const unsigned blocks = (unsigned)((long long)p.B * p.Hkv * (paired ? (ntk + 1) / 2 : ntk));
    if (p.block_mask)
        hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, true>), dim3(blocks), dim3(DkdvCfg<D>::THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, false>), dim3(blocks), dim3(DkdvCfg<D>::THREADS), 0, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dq(const BwdParams& p, hipStream_t stream) {
    constexpr int br = DqCfg<D>::BR;
    const unsigned blocks = (unsigned)((long long)p.B * p.Hq * ((p.N + br - 1) / br));
    if (p.block_mask)
        hipLaunchKernelGGL((fa_bwd_dq_kernel<D, true>), dim3(blocks), dim3(DqCfg<D>::THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((fa_bwd_dq_kernel<D, false>), dim3(blocks), dim3(DqCfg<D>::THREADS), 0, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_fused(const BwdParams& p, hipStream_t stream) {
    const unsigned blocks = (unsigned)((long long)p.B * p.Hkv * ((p.N + FusedCfg<D>::BK - 1) / FusedCfg<D>::BK));
    hipLaunchKernelGGL((fa_bwd_fused_kernel<D>), dim3(blocks), dim3(FusedCfg<D>::THREADS), 0, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dq_convert(const BwdParams& p, hipStream_t stream) {
    const long long n8 = (long long)p.B * p.Hq * p.N * D / 8;
    const unsigned blocks = (unsigned)((n8 + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(fa_bwd_dq_convert_kernel<D>, dim3(blocks), dim3(kThreads), 0, stream, p.dqacc,
                       (uint16_t*)p.dq, p.scale, n8);
    return hipGetLastError();
}

hipError_t launch_bwd_fused(const BwdParams& p, int d, hipStream_t stream) {
    return d == 64 ? launch_fused<64>(p, stream) : launch_fused<128>(p, stream);
}
hipError_t launch_bwd_dq_convert(const BwdParams& p, int d, hipStream_t stream) {
    return d == 64 ? launch_dq_convert<64>(p, stream) : launch_dq_convert<128>(p, stream);
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
hipError_t launch_bwd_dq_rows(const BwdParams& p, int d, hipStream_t stream) {
    BwdParams r = p;
    r.form_rows = 1;
    return d == 64 ? launch_dq<64>(r, stream) : launch_dq<128>(r, stream);
}

}  // namespace fa
