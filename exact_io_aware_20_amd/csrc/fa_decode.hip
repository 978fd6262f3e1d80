// Decode forward: a few new queries per head against a long key/value cache.
//
// What is computed is the forward of the plain definition with the queries placed
// at the end of the key sequence: query i of Nq sits at position Nk - Nq + i and,
// when causal, sees the keys up to that position (lecture summary, "衡量并优化推理":
// decoding reuses the cached keys and values of earlier tokens; "GPU 显存和注意力瓶颈":
// a token sees itself and earlier tokens).  The same lecture notes that token-by-token
// decoding moves much data for little arithmetic, so this path is bound by HBM
// bandwidth: every cached key and value is read once per call, and the design goal
// is to stream them at the memory's rate.
//
// gfx950 mapping:
//   * Grouped-query sharing (lecture summary, "减少缓存表示并验证草稿"): the G = Hq/Hkv
//     query heads of a KV head and their Nq queries are packed into one column set
//     of G*Nq rows, so each K/V byte is fetched once for the whole group.  Columns
//     are taken 32 at a time (a wave's MFMA columns); more than 32 packed rows use
//     further row blocks, which read the same K/V through L2.
//   * The key range is cut into splits of whole 64-key tiles so that the grid fills
//     the chip even for one sequence; each split is one single-wave workgroup with
//     its own 32 KB (d = 128) of LDS.  About 1024 splits are made, one wave per SIMD:
//     a fifth wave per CU (LDS would allow it) shares a SIMD with another and
//     measured slower than four.  Inside a split the per-tile
//     steps are those of the full-sequence forward: S^T = K Q^T on the matrix
//     cores, the lazily rescaled online softmax, O^T += V^T P^T.
//   * Each split writes its normalised partial output and its base-2 log-sum-exp (a
//     split with no key of its sequence writes only LSE = -inf, and is skipped);
//     a merge kernel combines the splits of a row with weights 2^(lse_s - lse),
//     the online softmax's rescaling applied to whole partial results (lecture
//     summary, "推导 FlashAttention 的在线 softmax").  With a single split the split
//     kernel writes the final bf16 O and natural-log LSE itself.
#include "fa_common.hpp"
#include "fa_fwd_tile.hpp"
#include "fa_launch.hpp"

namespace fa {

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8); the counters not named are left at their maximum.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Mask of a tile whose LDS row j holds key kb + j: keys below klo (a re-read of
// the previous tile), keys >= N and, when causal, keys after the column's position.
__device__ __forceinline__ void decode_mask(f32x16 (&s)[2], int kb, int klo, int pos, int N, int causal, int hh) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kb + 32 * h + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool vis = key >= klo && key < N && (!causal || key <= pos);
            s[h][r] = vis ? s[h][r] : kNegInf;
        }
}

template <int D, bool PAGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_decode_split_kernel(DecodeParams p) {
    using S = SwzTile<D, 1>;
    using Dma = TileDma<D, 1, 1, false>;   // global form: 8 % faster than the buffer form here (paged)
    constexpr int T = S::ELEMS;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T];
    uint16_t* kbuf = smem;
    uint16_t* vbuf = smem + T;

    const int lane = threadIdx.x;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // workgroup -> (KV head, split, row block); consecutive logical ids share an XCD
    int logical = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) logical = (logical & 7) * (nblk >> 3) + (logical >> 3);
    const int rb = logical % p.nrb;
    const int rest = logical / p.nrb;
    const int split = rest % p.nsplit;
    const int bh = rest / p.nsplit;   // b * Hkv + hkv
    const int b = bh / p.Hkv;
    const int hkv = bh - b * p.Hkv;
    const int G = p.Hq / p.Hkv;
    const int Nq = p.Nq;
    // this sequence's cached tokens (paged: its own length, at most the planned Nk)
    const int Nk = PAGED ? min(max(p.seq_lens[b], 0), p.Nk) : p.Nk;

    // this lane's query column: packed row r = (head within the group) * Nq + query
    const int r = rb * 32 + l32;
    const bool live = r < G * Nq;
    const int hl = live ? r / Nq : 0;
    const int qi = live ? r - hl * Nq : 0;
    const size_t qrow = ((size_t)b * p.Hq + (size_t)hkv * G + hl) * Nq + qi;
    const int pos = live ? Nk - Nq + qi : Nk - 1;   // position in the key sequence

    const uint16_t* Kp = (const uint16_t*)p.k;
    const uint16_t* Vp = (const uint16_t*)p.v;
    const uint16_t* Qr = (const uint16_t*)p.q + qrow * D;

    const int ntiles = (Nk + kDecodeTile - 1) / kDecodeTile;
    const int t0 = split * p.tiles_per_split;
    const int t1 = min(ntiles, t0 + p.tiles_per_split);
    if (t0 >= t1 && p.nsplit > 1) {
        // a split past this sequence's end (paged calls with mixed lengths): it sees
        // no key, so it records LSE = -inf only and the merge never reads its O
        if (live && hh == 0) p.part_lse[(size_t)split * p.B * p.Hq * Nq + qrow] = kNegInf;
        return;
    }

    u32x4 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qf[c] = live ? ld_global16(Qr + 16 * c + 8 * hh) : zero_u4();

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = zero16();
    float m_ref = kNegInf, l_part = 0.f;
    const float sl2 = p.scale_log2;

    // Tile t holds the 64 keys starting at kbase(t), read from element offset
    // tile_off(t) of the K and V arrays.  Contiguous cache: a ragged last tile is read
    // as the last 64 keys of the cache, its keys below 64 t (already in tile t-1)
    // masked, so that every load inside the loop is a whole tile; only a cache shorter
    // than one tile (a single tile, loaded before the loop) clamps its rows.  Paged
    // cache: a tile lies inside one page (page_size is a multiple of 64) and pages are
    // whole allocations, so every tile is read whole and keys >= Nk are masked; a
    // table entry outside [0, num_pages) is read as page 0 and its keys masked.
    auto kbase = [&](int t) {
        if (PAGED) return t * kDecodeTile;
        return Nk >= kDecodeTile ? min(t * kDecodeTile, Nk - kDecodeTile) : 0;
    };
    // The table entries of 64 consecutive pages of the sequence are held one per lane
    // and handed out by a lane shuffle, so that finding a tile's page needs no memory
    // round trip in front of its loads (one table read per 64 pages).
    int pchunk = -1, pent = 0;
    auto page_entry = [&](int pi) {
        const int c = pi >> 6;
        if (c != pchunk) {
            const int e = 64 * c + lane;
            pent = e < p.max_blocks ? p.block_table[(size_t)b * p.max_blocks + e] : -1;
            pchunk = c;
        }
        return __shfl(pent, pi & 63);
    };
    auto tile_off = [&](int t, bool& bad) -> size_t {
        if constexpr (PAGED) {
            const int key = t * kDecodeTile;
            int pg = page_entry(key / p.page_size);
            bad = (unsigned)pg >= (unsigned)p.num_pages;
            pg = bad ? 0 : pg;
            return (((size_t)pg * p.Hkv + hkv) * p.page_size + key % p.page_size) * D;
        } else {
            bad = false;
            return ((size_t)bh * Nk + kbase(t)) * D;
        }
    };
    // keys at or after this index may be invisible to some column of the block
    const int mask_from = p.causal ? Nk - Nq + 1 : Nk;

    Dma dma;
    dma.init(0, lane);

    // One tile in flight per operand: K(t+1) is fetched while tile t's softmax and
    // P.V run, V(t+1) while S(t+1) runs.  Loads retire in order, so "at most
    // Dma::PER outstanding" means the older of the two tiles in flight has landed.
    bool bad = false;
    size_t off = 0;
    if (t0 < t1) {
        off = tile_off(t0, bad);
        const int nvalid = PAGED ? kDecodeTile : Nk - kbase(t0);
        dma.issue(Kp + off, nvalid, kbuf, 0);
        dma.issue(Vp + off, nvalid, vbuf, 0);
    }
    for (int t = t0; t < t1; ++t) {
        const int klo = t * kDecodeTile;
        const int kb = kbase(t);
        const bool more = t + 1 < t1;
        bool bad1 = false;
        const size_t off1 = more ? tile_off(t + 1, bad1) : 0;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(Dma::PER));   // K(t) has landed
        f32x16 s[2];
        fwd_scores<D, 1>(kbuf, qf, s, l32, hh);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);              // K(t) fully read
        if (more) dma.issue_full(Kp + off1, kbuf, 0);
        if (kb < klo || kb + kDecodeTile > mask_from || bad)
            decode_mask(s, kb, klo, pos, bad ? kb : Nk, p.causal, hh);
        fwd_rescale<D>(s, o, m_ref, l_part, sl2);
        u32x4 pf[2][2];
        fwd_probs(s, m_ref, sl2, pf, l_part);
        if (more)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(Dma::PER));   // V(t) has landed
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        fwd_pv<D>(vbuf, pf, o, lane);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);              // V(t) fully read
        if (more) dma.issue_full(Vp + off1, vbuf, 0);
        off = off1;
        bad = bad1;
    }

    // ---- epilogue: l over the lane pair; a column that saw no key (possible only
    // in a split wholly after its position) has l = 0 and contributes nothing.
    const float lt = l_part + __shfl_xor(l_part, 32);
    if (!live) return;
    const bool any = lt > 0.f;
    const float inv = any ? 1.0f / lt : 0.f;
    if (p.nsplit == 1) {
        uint16_t* Or = (uint16_t*)p.o + qrow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2 v2 = {pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                  pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
                *(u32x2*)(Or + 32 * db + 8 * g + 4 * hh) = v2;
            }
        if (hh == 0) p.lse[qrow] = any ? (m_ref + __log2f(lt)) * kLn2 : kNegInf;
    } else {
        const size_t rows = (size_t)p.B * p.Hq * Nq;
        float* Or = p.part_o + ((size_t)split * rows + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 v4 = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                                  o[db][4 * g + 3] * inv};
                *(f32x4*)(Or + 32 * db + 8 * g + 4 * hh) = v4;
            }
        if (hh == 0) p.part_lse[(size_t)split * rows + qrow] = any ? m_ref + __log2f(lt) : kNegInf;
    }
}

// One workgroup per query row: the splits' base-2 LSEs give the row's maximum M and
// weights w_s = 2^(lse_s - M); O = sum_s w_s O_s / sum_s w_s and
// LSE = (M + log2 sum_s w_s) ln 2.  The LSEs are staged in LDS and turned into the
// weights there; then thread t adds the weighted
// partial outputs of splits t / (D/4), t / (D/4) + GR, ... for its four elements
// d = 4 (t % (D/4)) .. +3 (GR = 256 / (D/4) split groups).  The loop is unrolled so
// that a thread's loads are in flight together, and the split groups are summed
// through LDS at the end.  nsplit <= kDecodeTargetWgs (checked by the launcher).
template <int D>
__global__ __launch_bounds__(256) void fa_decode_merge_kernel(DecodeParams p) {
    constexpr int C4 = D / 4;        // float4 chunks of a row
    constexpr int GR = 256 / C4;     // split groups
    __shared__ float wts[kDecodeTargetWgs];
    __shared__ f32x4 red[GR][C4];
    __shared__ float rmax[4], rsum[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const size_t row = blockIdx.x;
    const size_t rows = (size_t)p.B * p.Hq * p.Nq;
    const int ns = p.nsplit;

    float mx = kNegInf;
    for (int s = tid; s < ns; s += 256) {
        const float l = p.part_lse[(size_t)s * rows + row];
        wts[s] = l;
        mx = fmaxf(mx, l);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) rmax[wave] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(rmax[0], rmax[1]), fmaxf(rmax[2], rmax[3]));
    if (M == kNegInf) {   // no split saw a key (a paged sequence shorter than its queries)
        if (tid < C4) {
            uint16_t* Or = (uint16_t*)p.o + row * D + 4 * tid;
            *(u32x2*)Or = u32x2{0u, 0u};
        }
        if (tid == 0) p.lse[row] = kNegInf;
        return;
    }
    float ws = 0.f;
    for (int s = tid; s < ns; s += 256) {
        const float w = fast_exp2(wts[s] - M);   // -inf -> 0
        wts[s] = w;
        ws += w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off);
    if (lane == 0) rsum[wave] = ws;
    __syncthreads();

    const int g = tid / C4, c = tid % C4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int s = g; s < ns; s += GR) {
        const float w = wts[s];
        if (w > 0.f) {   // a split that saw no key wrote no O
            const f32x4 x = *(const f32x4*)(p.part_o + ((size_t)s * rows + row) * D + 4 * c);
            acc += w * x;
        }
    }
    red[g][c] = acc;
    __syncthreads();
    if (tid < C4) {
        f32x4 x = red[0][tid];
#pragma unroll
        for (int j = 1; j < GR; ++j) x += red[j][tid];
        const float wt = rsum[0] + rsum[1] + rsum[2] + rsum[3];
        x *= 1.0f / wt;
        uint16_t* Or = (uint16_t*)p.o + row * D + 4 * tid;
        *(u32x2*)Or = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
        if (tid == 0) p.lse[row] = (M + __log2f(wt)) * kLn2;
    }
}

// ---------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------
template <int D>
static hipError_t launch_decode_d(const DecodeParams& p, int steps, bool paged, hipStream_t stream) {
    if (steps & kDecodeSplit) {
        const long long grid = (long long)p.B * p.Hkv * p.nrb * p.nsplit;
        if (paged)
            hipLaunchKernelGGL((fa_decode_split_kernel<D, true>), dim3((unsigned)grid), dim3(64), 0, stream, p);
        else
            hipLaunchKernelGGL((fa_decode_split_kernel<D, false>), dim3((unsigned)grid), dim3(64), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if ((steps & kDecodeMerge) && p.nsplit > 1) {
        if (p.nsplit > kDecodeTargetWgs) return hipErrorInvalidValue;   // the plan never makes more
        const long long rows = (long long)p.B * p.Hq * p.Nq;
        hipLaunchKernelGGL((fa_decode_merge_kernel<D>), dim3((unsigned)rows), dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, int d, int steps, bool paged, hipStream_t stream) {
    return d == 64 ? launch_decode_d<64>(p, steps, paged, stream) : launch_decode_d<128>(p, steps, paged, stream);
}

}  // namespace fa
