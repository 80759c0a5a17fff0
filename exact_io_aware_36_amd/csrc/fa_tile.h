// fa_tile.h -- LDS tile layout and MFMA operand access shared by the
// attention kernels (gfx950, wave64).
//
// A tile of R rows x D bf16 (D = 64 or 128) sits in LDS row-major with no
// padding, its 16-byte chunks permuted within each row by an XOR swizzle.
// Two access patterns read it:
//   * ld_row8: lane l reads 8 consecutive columns of row r (one 16-byte
//     chunk).  This is the MFMA operand when the tile's rows are the MFMA
//     rows (K for S^T = K Q^T, Q and dO in the backward).  16 lanes read 16
//     different rows at the same logical chunk.
//   * ld_tr8: the MFMA operand when the tile's COLUMNS are the MFMA rows and
//     the tile's rows run along k (V for O^T += V^T P^T, dO and Q for
//     dV^T, dK^T, K for dQ^T).  Two ds_read_b64_tr_b16 per operand; each
//     reads 4 tile rows x 64 bytes per half-wave and transposes in hardware.
// The swizzle makes both patterns free of bank conflicts (64 banks x 4 B):
// for D = 128 every row is one 256-byte bank window and the chunk index is
// XORed with ((r & 3) << 2 | (r >> 2) & 3); for D = 64 two rows share a
// window and the chunk index is XORed with ((r >> 1) & 1) << 2 | (r >> 2) & 3.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum of x over this lane and the lane 32 away (v_permlane32_swap)
__device__ __forceinline__ float pair_max(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int D>
__device__ __forceinline__ int swz(int row)
{
    static_assert(D == 64 || D == 128, "head dim");
    if constexpr (D == 128)
        return ((row & 3) << 2) | ((row >> 2) & 3);
    else
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// element offset of (row, col) in a swizzled tile; col % 4 == 0
template <int D>
__device__ __forceinline__ int toff(int row, int col)
{
    return row * D + ((((col >> 3) ^ swz<D>(row)) << 3) | (col & 7));
}

template <int D>
__device__ __forceinline__ bf16x8 ld_row8(const bf16 *t, int row, int col)
{
    return *(const bf16x8 *)(t + toff<D>(row, col));
}

// Transposed operand: lane l receives tile column col0 + (l & 31) at tile
// rows row0 + 4*(l >> 5) + {0,1,2,3, 8,9,10,11}, the k order that matches the
// register order of a 32x32 MFMA result (register 4g+e of lane half h holds
// result row 8g + 4h + e).  In one ds_read_b64_tr_b16, output lane 16G + i
// element e comes from the address of lane 16G + 4e + i/4, element i % 4, so
// lane s supplies row (s & 15) >> 2 and columns 4 (s & 3) .. +3 of its group.
template <int D>
__device__ __forceinline__ bf16x8 ld_tr8(const bf16 *t, int row0, int col0)
{
    const int lane = threadIdx.x & 63;
    const int r = row0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int c = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    typedef bf16x4 __attribute__((address_space(3))) lds_bf16x4;
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(t + toff<D>(r, c)));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(t + toff<D>(r + 8, c)));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Cooperative copy of a ROWS x D bf16 tile from global memory (rows of D
// contiguous elements) into a swizzled LDS tile, staged through registers so
// that the global loads of the next tile can be in flight during compute.
// Rows at or past `valid` are filled with zeros.
template <int ROWS, int D>
struct TileStage {
    static constexpr int CPR = D / 8;               // 16-byte chunks per row
    static constexpr int CH = ROWS * CPR / 256;     // chunks per thread
    static_assert(CH * 256 == ROWS * CPR, "tile must split evenly over 256 threads");
    bf16x8 r[CH];

    __device__ __forceinline__ void load(const bf16 *g, int valid)
    {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int cidx = threadIdx.x + 256 * i;
            const int row = cidx / CPR, col = (cidx % CPR) * 8;
            r[i] = row < valid ? *(const bf16x8 *)(g + (size_t)row * D + col) : bf16x8{};
        }
    }
    __device__ __forceinline__ void store(bf16 *t) const
    {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int cidx = threadIdx.x + 256 * i;
            const int row = cidx / CPR, col = (cidx % CPR) * 8;
            *(bf16x8 *)(t + toff<D>(row, col)) = r[i];
        }
    }
};

} // namespace fa
