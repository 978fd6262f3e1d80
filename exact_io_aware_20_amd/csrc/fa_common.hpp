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
constexpr int kWaves = 4;                 // waves per workgroup
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
// Staging of a 64-row bf16 tile [64][D] (row-major, rows >= nvalid read as zero)
// into LDS, in the natural layout [64][D + 8] and/or the transposed layout
// [D][64 + 4].  Each work item is 4 consecutive rows x 8 columns (four 16-byte
// global loads); the transposed copy is written as eight 8-byte stores.
// The paddings keep the fragment reads below free of bank conflicts.
// ---------------------------------------------------------------------------------
template <int D>
struct Tile64 {
    static constexpr int ROWS = 64;
    static constexpr int NSTR = D + 8;                 // natural row stride (elements)
    static constexpr int TSTR = ROWS + 4;              // transposed row stride (elements)
    static constexpr int N_ELEMS = ROWS * NSTR;
    static constexpr int T_ELEMS = D * TSTR;
    static constexpr int ITEMS = (D / 8) * (ROWS / 4);
    static constexpr int PER_THREAD = (ITEMS + kThreads - 1) / kThreads;
};

template <int D>
struct TileRegs {
    u32x4 r[Tile64<D>::PER_THREAD][4];
};

template <int D>
__device__ __forceinline__ void tile_load(TileRegs<D>& t, const uint16_t* src, int nvalid, int tid) {
    using T = Tile64<D>;
#pragma unroll
    for (int i = 0; i < T::PER_THREAD; ++i) {
        const int it = tid + i * kThreads;
        const int c = it % (D / 8);
        const int rq = it / (D / 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = rq * 4 + j;
            t.r[i][j] = (it < T::ITEMS && row < nvalid)
                            ? ld_global16(src + (size_t)row * D + c * 8)
                            : zero_u4();
        }
    }
}

template <int D>
__device__ __forceinline__ void tile_store_natural(const TileRegs<D>& t, uint16_t* dst, int tid) {
    using T = Tile64<D>;
#pragma unroll
    for (int i = 0; i < T::PER_THREAD; ++i) {
        const int it = tid + i * kThreads;
        if (it < T::ITEMS) {
            const int c = it % (D / 8);
            const int rq = it / (D / 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) *(u32x4*)(dst + (rq * 4 + j) * T::NSTR + c * 8) = t.r[i][j];
        }
    }
}

template <int D>
__device__ __forceinline__ void tile_store_transposed(const TileRegs<D>& t, uint16_t* dst, int tid) {
    using T = Tile64<D>;
#pragma unroll
    for (int i = 0; i < T::PER_THREAD; ++i) {
        const int it = tid + i * kThreads;
        if (it < T::ITEMS) {
            const int c = it % (D / 8);
            const int rq = it / (D / 8);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a = t.r[i][0][w], b = t.r[i][1][w];
                const uint32_t cc = t.r[i][2][w], d = t.r[i][3][w];
                // column 2w: low halves of the four rows; column 2w+1: high halves
                const u32x2 even = {(a & 0xffffu) | (b << 16), (cc & 0xffffu) | (d << 16)};
                const u32x2 odd = {(a >> 16) | (b & 0xffff0000u), (cc >> 16) | (d & 0xffff0000u)};
                *(u32x2*)(dst + (c * 8 + 2 * w) * T::TSTR + rq * 4) = even;
                *(u32x2*)(dst + (c * 8 + 2 * w + 1) * T::TSTR + rq * 4) = odd;
            }
        }
    }
}

// Fragment readers for the layouts above.
//  natural A/B fragment: row `row`, 8 columns starting at 16*c + 8*half
template <int D>
__device__ __forceinline__ u32x4 frag_natural(const uint16_t* base, int row, int c, int half) {
    return lds16(base + row * Tile64<D>::NSTR + 16 * c + 8 * half);
}
//  transposed fragment contracting over tile rows: column-of-tile `col` (an index
//  into d), tile rows kk + 4*half + {0..3} and kk + 8 + 4*half + {0..3}; this is
//  the (lane half, slot) -> k order that a C tile's registers 8*s16 .. 8*s16+7 have.
template <int D>
__device__ __forceinline__ u32x4 frag_transposed(const uint16_t* base, int col, int kk, int half) {
    const uint16_t* p = base + col * Tile64<D>::TSTR + kk + 4 * half;
    return cat(lds8(p), lds8(p + 8));
}

}  // namespace fa
