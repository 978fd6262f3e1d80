// Device-side building blocks shared by the forward and backward kernels (gfx950).
//
// Matrix-core conventions used throughout (wave64, v_mfma_f32_32x32x16_bf16):
//   A operand (32 x 16): lane l holds row (l % 32) and 8 values along k;
//   B operand (16 x 32): lane l holds column (l % 32) and 8 values along k;
//   the 8 k-slots of lanes 0-31 and of lanes 32-63 together cover the 16 k
//   indices, and A and B use the same slot -> k assignment, so any bijection of
//   (lane half, slot) onto k gives the same contraction.  We choose it per use.
//   C/D (32 x 32 fp32): lane l holds column (l % 32) and 16 rows
//   8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
// A C tile can therefore be fed back as an A operand (as its transpose) or as a
// B operand, contracting over its rows, without any cross-lane movement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kWaves = 4;                 // waves per workgroup of the elementwise kernels
constexpr int kThreads = kWave * kWaves;  // 256
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed bf16 pair (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ld_global16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 lds16(const uint16_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ u32x4 cat(const u32x2& a, const u32x2& b) {
    return u32x4{a[0], a[1], b[0], b[1]};
}

// Workgroup -> (head, row tile).  Workgroups are handed to the eight XCDs
// round-robin (id % 8); when both counts divide by 8, consecutive logical ids are
// gathered on one XCD so the row tiles of a head share that XCD's L2.  Logical ids
// then run over groups of `hg` heads (hg divides nhead/8), and within a group over
// row tiles first (heads of the group interleaved), in the order `reverse` asks
// (causal forward and dQ: last tiles first, since they have the most visible keys),
// so the heaviest tiles of the group start first and the lightest end the grid.
__device__ __forceinline__ void decode_item(int logical, int ntile, int nhead, bool reverse, int& head, int& tile,
                                            int hg = 1) {
    if (hg < 1 || ((nhead >> 3) % hg) != 0 || (nhead & 7) != 0) hg = 1;
    const int g = logical / (hg * ntile);
    const int r = logical - g * hg * ntile;
    const int t = r / hg;
    head = g * hg + (r - t * hg);
    tile = reverse ? ntile - 1 - t : t;
}
__device__ __forceinline__ void map_block(int bid, int nblk, int ntile, int nhead, bool reverse,
                                          int& head, int& tile, int hg = 1) {
    int logical = bid;
    if ((nblk & 7) == 0 && (nhead & 7) == 0) logical = (bid & 7) * (nblk >> 3) + (bid >> 3);
    decode_item(logical, ntile, nhead, reverse, head, tile, hg);
}

// ---------------------------------------------------------------------------------
// Swizzled natural tile [64][D] in LDS, filled by direct global->LDS loads
// (buffer_load_dwordx4 ... lds: lane L of a wave writes 16 bytes at base + 16*L).
// Row r's 16-byte chunk j lives at slot j ^ swz(r), with no padding.
//
// Two read patterns touch these tiles (bank = 4-byte word index mod 64):
//  * row fragments, ds_read_b128: lane l reads row 32q + l%32, chunk 2k + l/32.
//    The wave is served in four cycles of 16 lanes: the lanes of one half (l/32)
//    whose bits 2..4 have equal parity (measured on gfx950 with the
//    SQ_LDS_BANK_CONFLICT counter, one pair of active lanes at a time).  A cycle
//    is conflict-free when its lanes touch 16 distinct 16-byte slots of a
//    256-byte bank window.
//  * transposing reads, ds_read_b64_tr_b16 (tr_frag below): each half-wave cycle
//    reads 4 consecutive rows (aligned to 4) x 4 consecutive chunks (aligned to 4).
//    Conflict-free when the four rows put that 64-byte unit in four different
//    units of the bank window.
//   MODE 0 serves the fragment pattern only (r mod 16 for D = 128, two rows per
//   window for D = 64); MODE 1 serves both with a bit permutation of the row:
//   D = 128: bits (1,0 | 3,2) of r -> chunk bits (3,2 | 1,0); D = 64: r bits
//   1, 2, 3 -> chunk bits 2, 1, 0.  Both checked exhaustively on the CPU against
//   the cycle grouping above.
// ---------------------------------------------------------------------------------
template <int D, int MODE = 0>
struct SwzTile {
    static constexpr int CHUNKS = D / 8;          // 16-byte chunks per row
    static constexpr int ELEMS = 64 * D;          // bf16 elements per tile
    static constexpr int WAVE_LOADS = 64 * CHUNKS / kWave;   // wave-instructions per tile
    __device__ static __forceinline__ int swz(int r) {
        if (MODE == 0) return D == 128 ? (r & 15) : ((r >> 1) & 7);
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (((r & 2) << 1) | ((r >> 1) & 2) | ((r >> 3) & 1));
    }
    // element offset of (row, chunk)
    __device__ static __forceinline__ int at(int r, int j) { return r * D + ((j ^ swz(r)) << 3); }
};

typedef __attribute__((address_space(3))) void lds_void;

// Direct global->LDS loads go through buffer resources (buffer_load ... lds), not the
// global_load_lds form.  The compiler's wait insertion counts the global form against
// both the vector-memory and the LDS counters, and while one is in flight it turns every
// LDS wait into lgkmcnt(0).  Every loop that prefetches its next tile would then wait for
// all its outstanding fragment reads at each MFMA, not just the oldest.  With the buffer
// form those waits stay exact.  The builtin is called only from the two plain
// functions below: written inside a function template, a kernel template reaching it
// could lose its host-side launch stub without a diagnostic.
//
// Buffer resource over `bytes` bytes from `base` (raw, unformatted dword access; a read
// past the end returns zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// One direct load per lane of 16 (4) bytes at byte offset voff of r into LDS at dst +
// 16 (4) x lane; dst is wave-uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, voff, 0, 0, 0);
}
// The global form: 16 bytes per lane from the lane's own address.
__device__ __forceinline__ void dma16_global(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// Direct load of one 4-byte value per lane: lane l reads element min(l, nvalid - 1) of
// `src` into LDS at dst + 4 l.
__device__ __forceinline__ void dma_row_values(const float* src, int nvalid, void* dst, int lane) {
    dma4(tile_rsrc(src, nvalid * 4), (uint32_t)min(lane, nvalid - 1) * 4, dst);
}

// Direct loads of one 64-row tile: wave-instruction i (of WAVE_LOADS, spread over
// NWAVES waves) covers LDS chunk positions [64 i, 64 i + 64).  A wave's chunk
// positions do not change from tile to tile, so the per-lane source offsets are
// computed once and a full tile costs one load per chunk from a uniform base plus
// a 32-bit lane offset; only a ragged last tile (wave-uniform branch) clamps its
// rows.  `wave` must be below NWAVES.  BUF selects the buffer form (above) or the
// global_load_lds form.
template <int D, int MODE, int NWAVES, bool BUF = true>
struct TileDma {
    using S = SwzTile<D, MODE>;
    static constexpr int PER = (S::WAVE_LOADS + NWAVES - 1) / NWAVES;
    uint32_t off[PER];   // byte offset of this lane's 16-byte chunk within the global tile
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const uint32_t pos = (uint32_t)((wave + k * NWAVES) * 64 + lane);
            const uint32_t row = pos / S::CHUNKS;
            off[k] = (row * D + ((pos % S::CHUNKS) ^ (uint32_t)S::swz((int)row)) * 8) * 2;
        }
    }
    // all 64 rows of src are in bounds
    __device__ __forceinline__ void issue_full(const uint16_t* src, uint16_t* lds_tile, int wave) const {
        if constexpr (BUF) {
            const __amdgpu_buffer_rsrc_t r = tile_rsrc(src, 64 * D * 2);
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int i = wave + k * NWAVES;
                if (S::WAVE_LOADS % NWAVES == 0 || i < S::WAVE_LOADS) dma16(r, off[k], lds_tile + i * 64 * 8);
            }
        } else {
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int i = wave + k * NWAVES;
                if (S::WAVE_LOADS % NWAVES == 0 || i < S::WAVE_LOADS)
                    dma16_global((const char*)src + off[k], lds_tile + i * 64 * 8);
            }
        }
    }
    // rows at or past `nvalid` are read from row nvalid-1 (in bounds, never used)
    __device__ __forceinline__ void issue(const uint16_t* src, int nvalid, uint16_t* lds_tile, int wave) const {
        if (nvalid >= 64) {
            issue_full(src, lds_tile, wave);
        } else {
            const __amdgpu_buffer_rsrc_t r = tile_rsrc(src, nvalid * D * 2);
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int i = wave + k * NWAVES;
                if (S::WAVE_LOADS % NWAVES == 0 || i < S::WAVE_LOADS) {
                    const uint32_t row = off[k] / (2 * D);
                    const uint32_t last = (uint32_t)(nvalid - 1);
                    const uint32_t rr = row < last ? row : last;
                    const uint32_t voff = off[k] - (row - rr) * (2 * D);
                    if constexpr (BUF)
                        dma16(r, voff, lds_tile + i * 64 * 8);
                    else
                        dma16_global((const char*)src + voff, lds_tile + i * 64 * 8);
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------------
// A-operand fragment of X^T (D x 64) read from a natural MODE 1 tile X [64][D] with
// two ds_read_b64_tr_b16.  That instruction works on groups of 16 lanes: lane m of
// a group supplies the address of 4 consecutive bf16, and lane 4a+p receives
// element p of the values addressed by lanes a, a+4, a+8, a+12.  Lane m of group
// g = l/16 addresses row kk + 4(g/2) + m/4 (+8 for the second read), columns
// 32db + 16(g%2) + 4(m%4) .. +3, so lane l receives column d = 32db + l%32 of the 8
// rows kk + {4h .. 4h+3, 8+4h .. 8+4h+3}, h = l/32: the k-slot order in which a
// C tile's registers feed a B operand (see the convention at the top).
// ---------------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The transposing read goes through a helper whose pointer parameter is restrict:
// once inlined, the read carries alias-scope metadata.  Without it the compiler has
// no alias information for the read and waits for every direct global->LDS load
// still in flight (s_waitcnt vmcnt(0)) before it, which would stall each tile step
// on the prefetch of the next tiles.  Every kernel here waits for its direct loads
// explicitly (s_waitcnt, then a workgroup barrier) before any wave reads the LDS
// they fill, and never reads a buffer while a load into it is in flight, so the
// implicit wait is not needed for correctness.
__device__ __forceinline__ s16x4 tr_read_lds(const lds_s16x4* __restrict__ p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}
__device__ __forceinline__ u32x2 tr_read(const uint16_t* p) {
    return __builtin_bit_cast(u32x2, tr_read_lds((const lds_s16x4*)(p)));
}

template <int D>
__device__ __forceinline__ u32x4 tr_frag(const uint16_t* tile, int db, int kk, int lane) {
    using S = SwzTile<D, 1>;
    const int g = lane >> 4, m = lane & 15;
    const int row = kk + 4 * (g >> 1) + (m >> 2);
    const int col = 32 * db + 16 * (g & 1) + 4 * (m & 3);
    const u32x2 lo = tr_read(tile + S::at(row, col >> 3) + (col & 7));
    const u32x2 hi = tr_read(tile + S::at(row + 8, col >> 3) + (col & 7));
    return cat(lo, hi);
}

// Loop-hoisted LDS addressing.  Both swizzles depend on the row mod 16 only, so a
// fragment whose rows start at a multiple of 16 is a fixed per-lane offset plus a
// constant.  A kernel keeps the per-lane offsets, adds the current stage's LDS base
// once per tile, and hides that sum from the optimiser (opaque), so each constant
// stays an immediate of the read; without this the compiler hoisted one register per
// (fragment, constant) pair and re-added the stage base before every read.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ u32x2 tr_read_a(uint32_t a) {
    return __builtin_bit_cast(u32x2, tr_read_lds((const lds_s16x4*)(uintptr_t)a));
}
__device__ __forceinline__ u32x4 lds16_a(uint32_t a) {
    return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)a;
}

// Element offsets of the two tr_frag reads of column block db at kk = 0 (MODE 1 tile).
template <int D>
struct TrOffsets {
    uint32_t off[D / 32][2];
    __device__ __forceinline__ void init(int lane) {
        using S = SwzTile<D, 1>;
        const int g = lane >> 4, m = lane & 15;
        const int row = 4 * (g >> 1) + (m >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int col = 32 * db + 16 * (g & 1) + 4 * (m & 3);
            off[db][0] = (uint32_t)(S::at(row, col >> 3) + (col & 7));
            off[db][1] = (uint32_t)(S::at(row + 8, col >> 3) + (col & 7));
        }
    }
};

// tr_frag of the MODE 1 tile at LDS byte address `base`, for kk a multiple of 16
template <int D>
struct TrAddr {
    uint32_t a[D / 32][2];
    __device__ __forceinline__ TrAddr(const TrOffsets<D>& o, uint32_t base) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            a[db][0] = opaque(base + 2 * o.off[db][0]);
            a[db][1] = opaque(base + 2 * o.off[db][1]);
        }
    }
    __device__ __forceinline__ u32x4 frag(int db, int kk) const {
        return cat(tr_read_a(a[db][0] + 2 * kk * D), tr_read_a(a[db][1] + 2 * kk * D));
    }
};

// The two tr_frag reads of one column block `db` chosen at run time (a wave-dependent
// index into TrAddr's per-block array would force that array into scratch memory):
// element offsets at kk = 0, then a per-tile opaque base as in TrAddr.
template <int D>
struct TrColOffsets {
    uint32_t off[2];
    __device__ __forceinline__ void init(int lane, int db) {
        using S = SwzTile<D, 1>;
        const int g = lane >> 4, m = lane & 15;
        const int row = 4 * (g >> 1) + (m >> 2);
        const int col = 32 * db + 16 * (g & 1) + 4 * (m & 3);
        off[0] = (uint32_t)(S::at(row, col >> 3) + (col & 7));
        off[1] = (uint32_t)(S::at(row + 8, col >> 3) + (col & 7));
    }
};
template <int D>
struct TrColAddr {
    uint32_t a[2];
    __device__ __forceinline__ TrColAddr(const TrColOffsets<D>& o, uint32_t base) {
        a[0] = opaque(base + 2 * o.off[0]);
        a[1] = opaque(base + 2 * o.off[1]);
    }
    __device__ __forceinline__ u32x4 frag(int kk) const {
        return cat(tr_read_a(a[0] + 2 * kk * D), tr_read_a(a[1] + 2 * kk * D));
    }
};

// ---------------------------------------------------------------------------------
// Block-sparse layouts: a 0/1 byte matrix over 64 x 64 blocks of (query, key)
// positions, nb x nb with nb = ceil(N / 64), shared by every (batch, head).  A
// workgroup first compacts the tiles it has to visit into an LDS list.
// ---------------------------------------------------------------------------------
constexpr int kSparseBlock = 64;
constexpr int kSparseMaxBlocks = 2048;   // N <= 131072
constexpr uint32_t kSparseTileMask = (1u << 20) - 1;

// One wave, lanes over the candidates u in [begin, end): bits(u) returns a small bit
// set (which of the workgroup's blocks see candidate u; 0 = none).  Entries
// u | bits << 20 are appended to `list` in increasing u; returns their number (the
// same in every lane).  Candidates outside [begin, end) are never listed, so callers
// narrow the range to what the causal rule leaves.  bits(u) must stay in bounds for
// any u in the range (it is called for clamped candidates too).  BATCH groups of 64
// candidates are evaluated before the first ballot; with a branch-free bits(u) their
// layout reads are in flight together.
template <int BATCH = 4, typename F>
__device__ __forceinline__ int compact_tiles(uint32_t* list, int begin, int end, int lane, F bits) {
    int cnt = 0;
    for (int base = begin; base < end; base += BATCH * kWave) {
        uint32_t b[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int u = base + i * kWave + lane;
            const uint32_t bu = bits(min(u, end - 1));   // evaluated for every lane: no branch
            b[i] = u < end ? bu : 0u;
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int u = base + i * kWave + lane;
            const uint64_t m = __ballot(b[i] != 0u);
            const int below =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            if (b[i] != 0u) list[cnt + below] = (uint32_t)u | (b[i] << 20);
            cnt += __popcll(m);
        }
    }
    return cnt;
}

}  // namespace fa
