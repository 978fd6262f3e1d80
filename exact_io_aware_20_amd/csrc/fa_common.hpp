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
__device__ __forceinline__ u32x2 lds8(const uint16_t* p) { return *(const u32x2*)p; }
__device__ __forceinline__ u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ u32x4 cat(const u32x2& a, const u32x2& b) {
    return u32x4{a[0], a[1], b[0], b[1]};
}

// Workgroup -> (head, row tile).  Workgroups are handed to the eight XCDs
// round-robin (id % 8); when both counts divide by 8, consecutive logical ids are
// gathered on one XCD so all row tiles of a head share that XCD's L2.  Within a
// head, row tiles are issued in the order `reverse` asks (causal forward and dQ:
// last tiles first, since they have the most visible keys).
__device__ __forceinline__ void map_block(int bid, int nblk, int ntile, int nhead, bool reverse,
                                          int& head, int& tile) {
    int logical = bid;
    if ((nblk & 7) == 0 && (nhead & 7) == 0) logical = (bid & 7) * (nblk >> 3) + (bid >> 3);
    head = logical / ntile;
    int t = logical - head * ntile;
    tile = reverse ? ntile - 1 - t : t;
}

// ---------------------------------------------------------------------------------
// Swizzled natural tile [64][D] in LDS, filled by direct global->LDS loads
// (global_load_lds_dwordx4: lane L of a wave writes 16 bytes at base + 16*L).
// Row r's 16-byte chunk j lives at slot j ^ swz(r), with no padding.
//
// ds_read_b128 serves a wave in four cycles of 16 lanes: the lanes of one half
// (l / 32) whose bits 2..4 have equal parity (measured on gfx950 with the
// SQ_LDS_BANK_CONFLICT counter, one pair of active lanes at a time).  A cycle is
// conflict-free when its 16 lanes touch 16 distinct 16-byte slots of a 256-byte
// bank window.  The swizzles are chosen for that grouping:
//   MODE 0: fragment reads (lane l: row 32q + l%32, chunk 2k + l/32);
//   MODE 1: fragment reads and transposing reads (lane l of a wave: rows 4(l%16)+j
//           of chunk c0 + l/16).  For D = 128 the Gray code r ^ r/2 serves both
//           with no conflict; for D = 64 (two rows per bank window) the rows of a
//           transposing read share a parity, so a 2-way conflict there is the
//           least any row swizzle allows, and r ^ r/4 reaches it.
// ---------------------------------------------------------------------------------
template <int D, int MODE = 0>
struct SwzTile {
    static constexpr int CHUNKS = D / 8;          // 16-byte chunks per row
    static constexpr int ELEMS = 64 * D;          // bf16 elements per tile
    static constexpr int WAVE_LOADS = 64 * CHUNKS / kWave;   // wave-instructions per tile
    __device__ static __forceinline__ int swz(int r) {
        if (MODE == 0) return D == 128 ? (r & 15) : ((r >> 1) & 7);
        return D == 128 ? ((r ^ (r >> 1)) & 15) : ((r ^ (r >> 2)) & 7);
    }
    // element offset of (row, chunk)
    __device__ static __forceinline__ int at(int r, int j) { return r * D + ((j ^ swz(r)) << 3); }
};

typedef __attribute__((address_space(3))) void lds_void;

// Returns x unchanged, but opaque to the optimiser: per-lane address arithmetic
// that depends on it is recomputed where it is used instead of being hoisted out
// of the main loop and kept live (which would spill under full register use).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Issue the direct loads of one 64-row tile: wave-instruction i (of WAVE_LOADS)
// covers LDS chunk positions [64 i, 64 i + 64).  Rows at or past `nvalid` are
// read from row nvalid-1 instead (always in bounds; callers mask those rows or
// give them zero weight).
template <int D, int MODE, int NWAVES>
__device__ __forceinline__ int swz_tile_issue(const uint16_t* src, int nvalid, uint16_t* lds_tile,
                                              int wave, int lane) {
    using S = SwzTile<D, MODE>;
    lane = opaque(lane);
    int issued = 0;
#pragma unroll
    for (int k = 0; k < (S::WAVE_LOADS + NWAVES - 1) / NWAVES; ++k) {
        const int i = wave + k * NWAVES;
        if (i < S::WAVE_LOADS) {
            const int pos = i * 64 + lane;
            const int r = pos / S::CHUNKS;
            const int slot = pos % S::CHUNKS;
            const int j = slot ^ S::swz(r);
            const int rr = r < nvalid ? r : nvalid - 1;
            __builtin_amdgcn_global_load_lds(src + (size_t)rr * D + j * 8,
                                             (lds_void*)(lds_tile + i * 64 * 8), 16, 0, 0);
            ++issued;
        }
    }
    return issued;
}

// ---------------------------------------------------------------------------------
// Transposed tile with key-permuted columns: [D][64 + 8] bf16.  Column position of
// key k within its 16-key block: 8*((k/4)&1) + 4*((k/8)&1) + (k%4), so that the 8
// keys one lane feeds to a 32x32x16 MFMA (k-slot order 4h+{0..3}, 8+4h+{0..3}) are
// contiguous and a fragment is one 16-byte read.
// ---------------------------------------------------------------------------------
template <int D>
struct PermT {
    static constexpr int STR = 64 + 8;
    static constexpr int ELEMS = D * STR;
    static constexpr int ITEMS = (D / 8) * 16;   // 4 keys x 8 columns per item
};

__device__ __forceinline__ int perm_pos4(int kq) {   // position of key 4*kq
    return 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq >> 1) & 1);
}

// Items are numbered key-quad fastest: the 16 lanes of a store cover one row's 64
// keys, so a wave's eight-byte stores hit distinct banks.
template <int D>
__device__ __forceinline__ void permt_load(u32x4 (&r)[4], const uint16_t* src, int nvalid, int item) {
    const int kq = item % 16, c = item / 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = kq * 4 + j;
        r[j] = row < nvalid ? ld_global16(src + (size_t)row * D + c * 8) : zero_u4();
    }
}

template <int D>
__device__ __forceinline__ void permt_store(const u32x4 (&r)[4], uint16_t* dst, int item) {
    const int kq = item % 16, c = item / 16;
    const int col = perm_pos4(kq);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t a = r[0][w], b = r[1][w], cc = r[2][w], d = r[3][w];
        const u32x2 even = {(a & 0xffffu) | (b << 16), (cc & 0xffffu) | (d << 16)};
        const u32x2 odd = {(a >> 16) | (b & 0xffff0000u), (cc >> 16) | (d & 0xffff0000u)};
        *(u32x2*)(dst + (c * 8 + 2 * w) * PermT<D>::STR + col) = even;
        *(u32x2*)(dst + (c * 8 + 2 * w + 1) * PermT<D>::STR + col) = odd;
    }
}

// Transpose one item (4 rows x 8 columns) from a MODE 1 swizzled natural tile in
// LDS into the permuted transposed layout.  Rows >= nvalid are written as zero, so
// stale or clamped rows contribute nothing to the contractions over rows.
template <int D, int MODE = 1>
__device__ __forceinline__ void permt_from_lds(const uint16_t* src, uint16_t* dst, int nvalid, int item) {
    using S = SwzTile<D, MODE>;
    item = opaque(item);
    const int kq = item % 16, c = item / 16;
    u32x4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = kq * 4 + j;
        r[j] = lds16(src + S::at(row, c));
        if (row >= nvalid) r[j] = zero_u4();
    }
    permt_store<D>(r, dst, item);
}

// Fragment of the permuted transposed tile: row `row` (an index into d), the 8
// keys kk + {4h..4h+3, 8+4h..8+4h+3} (kk a multiple of 16).
template <int D>
__device__ __forceinline__ u32x4 permt_frag(const uint16_t* base, int row, int kk, int half) {
    return lds16(base + row * PermT<D>::STR + kk + 8 * half);
}

}  // namespace fa
