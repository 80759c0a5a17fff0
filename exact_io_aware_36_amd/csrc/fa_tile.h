// fa_tile.h -- LDS tile layout and MFMA operand access shared by the
// attention kernels (gfx950, wave64).
//
// A tile of R rows x D bf16 (D = 64, 128 or 256) sits in LDS row-major with no
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
// XORed with ((r & 3) << 2 | (r >> 2) & 3); for D = 256 a row is two whole
// windows and the same XOR is applied to the low four bits of the chunk
// index; for D = 64 two rows share a window and the chunk index is XORed
// with ((r >> 1) & 1) << 2 | (r >> 2) & 3.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
    static_assert(D == 64 || D == 128 || D == 256, "head dim");
    if constexpr (D >= 128)   // D = 256: two bank windows per row, same low-bit XOR
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

// Buffer resource over one head's [N][D] bf16 rows: loads past the last row
// return zeros (the hardware range check), so ragged tiles need no
// predication.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const bf16 *base, int rows, int D)
{
    // byte count computed unsigned: rows * D * 2 may reach 2^32 - 2 (the
    // hardware field is 32-bit unsigned)
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0,
                                            (int)((unsigned)rows * (unsigned)D * 2u), 0x00020000);
}

// wave index as a scalar, so that branches on it are uniform
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Cooperative copy of a ROWS x D bf16 tile (rows row0 .. row0+ROWS-1 of a
// head) into a swizzled LDS tile, staged through registers so that the
// global loads of the next tile are in flight during compute.  Rows past the
// head's end read as zeros.
template <int ROWS, int D>
struct TileStage {
    static constexpr int CPR = D / 8;               // 16-byte chunks per row
    static constexpr int CH = ROWS * CPR / 256;     // chunks per thread
    static_assert(CH * 256 == ROWS * CPR, "tile must split evenly over 256 threads");
    bf16x8 r[CH];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int row0)
    {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int cidx = threadIdx.x + 256 * i;
            const int row = cidx / CPR, col = (cidx % CPR) * 8;
            const unsigned off = ((unsigned)(row0 + row) * (unsigned)D + (unsigned)col) * 2u;
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
            r[i] = __builtin_bit_cast(bf16x8, v);
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

// one 16-byte-per-lane buffer->LDS load (wrapped in a plain device function:
// used directly inside kernel templates, the builtin kept the host pass from
// emitting those kernels' handles)
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rs, bf16 *lds, unsigned voff,
                                                int soff)
{
    typedef void __attribute__((address_space(3))) lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)lds, 16, voff, soff, 0, 0);
}

// one 4-byte-per-lane buffer->LDS load: 64 floats per wave instruction
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t rs, float *lds, unsigned voff,
                                               int soff)
{
    typedef void __attribute__((address_space(3))) lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)lds, 4, voff, soff, 0, 0);
}

// Direct global -> LDS tile copy (buffer_load_dwordx4 ... lds, no register
// staging).  One such load writes the 16 bytes of lane L at LDS address
// M0 + 16 L, so each wave instruction fills 1 KB of the tile in physical
// order; the swizzle is applied on the global side: the lane that owns
// physical chunk pc of row r loads logical chunk pc ^ swz(r).  The WAVES
// waves of the workgroup split the tile's 1 KB segments round-robin.  The
// copy is asynchronous: wait on vmcnt, then barrier, before reading.
template <int ROWS, int D, int WAVES>
struct TileDma {
    static constexpr int CPR = D / 8;                      // 16-byte chunks per row
    static constexpr int SEGS = ROWS * CPR / 64;           // 1 KB segments per tile
    static constexpr int PER_WAVE = SEGS / WAVES;
    static_assert(PER_WAVE * WAVES == SEGS, "tile must split evenly over the waves");
    unsigned voff[PER_WAVE];                               // per-lane byte offsets within the tile

    __device__ __forceinline__ void init(int wave)
    {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int chunk = (wave + WAVES * i) * 64 + lane;      // physical chunk in tile
            const int row = chunk / CPR, pc = chunk % CPR;
            voff[i] = (unsigned)((row * D + ((pc ^ swz<D>(row)) << 3)) * 2);
        }
    }
    // copy rows row0 .. row0+ROWS-1 of the head behind rs into tile t
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int row0, bf16 *t, int wave) const
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i)
            buffer_to_lds16(rs, t + (wave + WAVES * i) * 512, voff[i], (int)((unsigned)row0 * (unsigned)D * 2u));
    }
};

// wait until every vector-memory load of this wave (including LDS DMA) landed
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

} // namespace fa
