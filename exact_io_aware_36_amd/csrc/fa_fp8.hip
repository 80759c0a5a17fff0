// fa_fp8.hip -- block-quantised FP8 attention forward for gfx950, and the
// quantiser that prepares its inputs.
//
// The pages describe FP8 attention as block-quantised FP8 matrix products
// with dynamic scaling ("FlashAttention: Mathematical Foundations, IO-Aware
// Tiling, Online Softmax, and Recomputation Dynamics", section
// "FlashAttention-3", item on low-precision FP8 support), with block
// quantisation and incoherent processing ("Attention" chapter of
// learn-kernels.com, paragraph on Hopper).  Format and scale rules used here:
// OCP E4M3 ("FN", largest finite 448) rounded to nearest even by
// v_cvt_pk_fp8_f32; each block's largest magnitude maps to 448
// (inv = 448 / amax, code = E4M3(x * inv), descale = amax / 448, fp32);
// Q and K in blocks of 128 rows of one (b, h), V in one block per (b, h) so
// that its scale factors out of the P V sum.  Incoherent processing
// multiplies Q and K by the same orthogonal R = diag(signs) H_d / sqrt(d)
// (H_d the Sylvester Hadamard matrix): Q R (K R)^T = Q K^T, while outliers
// are spread over all d coordinates before rounding.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.f;
constexpr float TAU8 = 8.f;     // lazy-rescale threshold (log2 units)
constexpr float kPassLimit8 = 256.f;   // 2^TAU8

// ---------------------------------------------------------------------------
// Quantiser.  One workgroup (256 threads) per 128-row block of one (b, h).
// A row is D/8 lanes wide (8 elements per lane); 256 / (D/8) rows per pass.
//
// The rotation is the fast Walsh-Hadamard transform in fp32: signs first,
// then butterflies of widths 1, 2, 4 inside a lane and 8, 16, ... across the
// row's lanes, each pair (a, b) -> (a + b, a - b) with a the lower index,
// then the multiply by rs = 1/sqrt(d).
template <int D, bool ROT>
struct QuantRows {
    static constexpr int LPR = D / 8;
    static constexpr int RPP = 256 / LPR;
    static constexpr int PASSES = 128 / RPP;
    float v[PASSES][8];

    __device__ __forceinline__ void load(const bf16 *x, int row0, int nrows, const float *signs,
                                         float rs)
    {
        const int t = threadIdx.x, c = t % LPR;
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int r = ps * RPP + t / LPR;
            u32x4 w = {0, 0, 0, 0};
            if (r < nrows)
                w = *(const u32x4 *)(x + (size_t)(row0 + r) * D + 8 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned wi = w[i];
                v[ps][2 * i] = __uint_as_float(wi << 16);
                v[ps][2 * i + 1] = __uint_as_float(wi & 0xFFFF0000u);
            }
        }
        if constexpr (ROT) {
            float sg[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                sg[i] = signs[8 * c + i];
#pragma unroll
            for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    v[ps][i] *= sg[i];
                // widths 1, 2, 4: inside the lane
#pragma unroll
                for (int h = 1; h < 8; h *= 2)
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if ((i & h) == 0) {
                            const float a = v[ps][i], b = v[ps][i + h];
                            v[ps][i] = a + b;
                            v[ps][i + h] = a - b;
                        }
                // widths 8, 16, ...: lane ^ m within the row's lanes
#pragma unroll
                for (int m = 1; m < LPR; m *= 2) {
                    const bool upper = (t & m) != 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float o = __shfl_xor(v[ps][i], m);
                        v[ps][i] = upper ? o - v[ps][i] : v[ps][i] + o;
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    v[ps][i] *= rs;
            }
        }
    }

    // largest magnitude over the workgroup's rows (every thread gets it)
    __device__ __forceinline__ float block_amax(float *red) const
    {
        float a = 0.f;
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                a = fmaxf(a, fabsf(v[ps][i]));
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            a = fmaxf(a, __shfl_xor(a, off));
        if ((threadIdx.x & 63) == 0)
            red[threadIdx.x >> 6] = a;
        __syncthreads();
        a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        return a;
    }

    // codes of pass ps as two dwords (elements 0..3, 4..7)
    __device__ __forceinline__ u32x2 codes(int ps, float inv) const
    {
        u32x2 out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int w = 0;
            w = __builtin_amdgcn_cvt_pk_fp8_f32(v[ps][4 * h] * inv, v[ps][4 * h + 1] * inv, w, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(v[ps][4 * h + 2] * inv, v[ps][4 * h + 3] * inv, w, true);
            out[h] = (unsigned)w;
        }
        return out;
    }
};

struct QuantArgs {
    const bf16 *x;
    uint8_t *x8;
    float *descale;     // [B][H][nblk] (per-block) or [B][H] (per head)
    float *amax_ws;     // per-head mode: [B][H][nblk] block maxima
    const float *signs; // nullable
    float rs;           // 1/sqrt(d) as fp32
    int B, H, N, nblk;
};

// pass 1 of the per-head mode: each block's largest magnitude
template <int D, bool ROT>
__global__ __launch_bounds__(256) void quant_amax_kernel(QuantArgs p)
{
    __shared__ float red[4];
    const int blk = blockIdx.x % p.nblk, bh = blockIdx.x / p.nblk;
    const int row0 = blk * 128, nrows = min(128, p.N - row0);
    QuantRows<D, ROT> q;
    q.load(p.x + (size_t)bh * p.N * D, row0, nrows, p.signs, p.rs);
    const float a = q.block_amax(red);
    if (threadIdx.x == 0)
        p.amax_ws[blockIdx.x] = a;
}

// quantise one block; PER_HEAD takes the maximum over the head's block maxima
template <int D, bool ROT, bool PER_HEAD, bool TRANSPOSE>
__global__ __launch_bounds__(256) void quant_kernel(QuantArgs p)
{
    __shared__ float red[4];
    __shared__ float head_amax;
    __shared__ uint8_t tile[TRANSPOSE ? D * 128 : 1];
    const int blk = blockIdx.x % p.nblk, bh = blockIdx.x / p.nblk;
    const int row0 = blk * 128, nrows = min(128, p.N - row0);
    QuantRows<D, ROT> q;
    q.load(p.x + (size_t)bh * p.N * D, row0, nrows, p.signs, p.rs);
    float amax;
    if constexpr (PER_HEAD) {
        if (threadIdx.x < 64) {
            float a = 0.f;
            for (int i = threadIdx.x; i < p.nblk; i += 64)
                a = fmaxf(a, p.amax_ws[(size_t)bh * p.nblk + i]);
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1)
                a = fmaxf(a, __shfl_xor(a, off));
            if (threadIdx.x == 0)
                head_amax = a;
        }
        __syncthreads();
        amax = head_amax;
    } else {
        amax = q.block_amax(red);
    }
    const float inv = amax > 0.f ? kE4M3Max / amax : 1.f;
    const float ds = amax > 0.f ? amax / kE4M3Max : 1.f;
    if (threadIdx.x == 0) {
        if constexpr (PER_HEAD) {
            if (blk == 0)
                p.descale[bh] = ds;
        } else {
            p.descale[blockIdx.x] = ds;
        }
    }
    constexpr int LPR = QuantRows<D, ROT>::LPR, RPP = QuantRows<D, ROT>::RPP;
    const int t = threadIdx.x, c = t % LPR;
    if constexpr (!TRANSPOSE) {
        uint8_t *out = p.x8 + (size_t)bh * p.N * D;
#pragma unroll
        for (int ps = 0; ps < QuantRows<D, ROT>::PASSES; ++ps) {
            const int r = ps * RPP + t / LPR;
            const u32x2 w = q.codes(ps, inv);
            if (r < nrows)
                *(u32x2 *)(out + (size_t)(row0 + r) * D + 8 * c) = w;
        }
    } else {
        // stage as [D][128] bytes, then write 16-byte pieces of each d row
#pragma unroll
        for (int ps = 0; ps < QuantRows<D, ROT>::PASSES; ++ps) {
            const int r = ps * RPP + t / LPR;
            const u32x2 w = q.codes(ps, inv);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                tile[(8 * c + i) * 128 + r] = (uint8_t)(w[i / 4] >> (8 * (i % 4)));
        }
        __syncthreads();
        uint8_t *out = p.x8 + (size_t)bh * D * p.N;
        for (int k = t; k < D * 8; k += 256) {
            const int d = k / 8, part = k % 8;
            if (part * 16 < nrows)
                *(u32x4 *)(out + (size_t)d * p.N + row0 + part * 16) = *(const u32x4 *)(tile + d * 128 + part * 16);
        }
    }
}

// ---------------------------------------------------------------------------
// FP8 forward.  The schedule of the bf16 forward (128 queries per workgroup,
// 4 waves x 32, 64-key tiles through two LDS stages, S^T = K Q^T so that a
// lane owns one query, lazy rescaling), on v_mfma_f32_32x32x64_f8f6f4 with
// both operands E4M3: one instruction contracts 64 bytes of k per lane pair.
//
// Operand slots.  In that instruction lane l supplies row (A) or column (B)
// l % 32 and 32 k-slots (32 bytes); the A slot (lane half h, byte j) meets
// the B slot with the same (h, j).  So any assignment of contraction indices
// to slots works as long as both operands use it:
//   S^T = K Q^T: slot (h, j) of k-step st is head coordinate 64 st + 32 h + j
//     (32 contiguous bytes of the row, for K and for Q alike);
//   O^T += V^T P^T: slot (h, j) is key (j / 16) * 32 + 16 h + (j % 16).
// The K rows are loaded in a permuted order -- A row m of a 32-key chunk is
// key 16 ((m >> 2) & 1) + 4 (m >> 3) + (m & 3) -- so that result register r
// of lane half h holds key 16 h + r: the 32 probabilities a lane holds over
// a 64-key tile are then exactly its 32 P^T slots, packed by
// v_cvt_pk_fp8_f32, and the matching V^T slots are two 16-byte runs of one
// V^T row.  V^T is stored transposed ([d][N] per head) by the quantiser.
//
// Scales: S = (q8 . k8) dq dk, so the tile's exp2 multiplier is
// scale log2(e) dq dk (dq of the workgroup's 128-row block, dk of the tile's
// 128-key block); V's per-head scale multiplies O once at the end.
struct Fp8FwdArgs {
    const uint8_t *q8, *k8, *v8t;
    const float *qs, *ks, *vs;
    bf16 *o;
    float *lse;
    int B, H, N, nblk;
    float c_log2;
    const int32_t *kv_lens;
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 16-byte chunk swizzles (conflict-free for the operand reads above)
template <int D>
__device__ __forceinline__ int kswz(int r)
{
    if constexpr (D == 128)
        return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
    else
        return ((r >> 2) & 1) | (((r >> 4) & 1) << 1);
}
__device__ __forceinline__ int vswz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ u32x4 lds16(const uint8_t *p) { return *(const u32x4 *)p; }

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(Fp8FwdArgs p)
{
    constexpr int BR = 128, BC = 64;
    constexpr int KSTEPS = D / 64;       // 64-byte k-steps of S^T
    constexpr int NDB = D / 32;          // 32-wide d blocks of O^T
    constexpr int KCH = D / 16;          // 16-byte chunks per K row
    constexpr int KSEG = BC * KCH / 64;  // 1 KB DMA segments per K tile
    constexpr int VSEG = D * 4 / 64;     // per V^T tile (rows of 64 bytes)
    static_assert(KSEG % 4 == 0 || KSEG < 4, "segments");

    __shared__ __attribute__((aligned(1024))) uint8_t k0s[BC * D];
    __shared__ __attribute__((aligned(1024))) uint8_t v0s[D * BC];
    __shared__ __attribute__((aligned(1024))) uint8_t k1s[BC * D];
    __shared__ __attribute__((aligned(1024))) uint8_t v1s[D * BC];

    const int N = p.N;
    const int n_qblk = (N + BR - 1) / BR;
    const int total = p.B * p.H * n_qblk;
    int bh, qb;
    if (CAUSAL) {
        causal_item(blockIdx.x, p.B * p.H, n_qblk, l2_group(N, 2 * D), bh, qb);
        qb = n_qblk - 1 - qb;                // rank 0 = the last block: longest rows
    } else {
        const int w = xcd_remap(blockIdx.x, total);
        bh = w / n_qblk;
        qb = w % n_qblk;
    }
    const int b = bh / p.H;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int q0 = qb * BR;
    const int wq0 = q0 + wave * 32;
    const int qrow = wq0 + l32;

    int kv_len = N;
    if (p.kv_lens) {
        kv_len = p.kv_lens[b];
        kv_len = kv_len < 0 ? 0 : (kv_len > N ? N : kv_len);
    }
    int kv_end = kv_len;
    if (CAUSAL)
        kv_end = min(kv_end, q0 + BR);
    const int n_tiles = (kv_end + BC - 1) / BC;

    const uint8_t *qh = p.q8 + (size_t)bh * N * D;
    const auto krs = __builtin_amdgcn_make_buffer_rsrc((void *)(p.k8 + (size_t)bh * N * D), (short)0,
                                                       N * D, 0x00020000);
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void *)(p.v8t + (size_t)bh * D * N), (short)0,
                                                       D * N, 0x00020000);
    const float c_q = p.c_log2 * p.qs[(size_t)bh * p.nblk + qb];
    const float *ksc = p.ks + (size_t)bh * p.nblk;

    // Q operands: 32 contiguous bytes of the row per k-step and lane half
    i32x8 qreg[KSTEPS];
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
        u32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
        if (qrow < N) {
            a = *(const u32x4 *)(qh + (size_t)qrow * D + st * 64 + 32 * hf);
            c = *(const u32x4 *)(qh + (size_t)qrow * D + st * 64 + 32 * hf + 16);
        }
        qreg[st] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    }

    // DMA offsets: the lane owning physical chunk pc of a tile loads the
    // logical chunk pc ^ swizzle(row)
    unsigned kvoff[(KSEG + 3) / 4], vvoff[(VSEG + 3) / 4];
#pragma unroll
    for (int i = 0; i < (KSEG + 3) / 4; ++i) {
        const int pc = (wave + 4 * i) * 64 + lane;
        const int row = pc / KCH, ph = pc % KCH;
        kvoff[i] = (unsigned)(row * D + ((ph ^ kswz<D>(row)) << 4));
    }
#pragma unroll
    for (int i = 0; i < (VSEG + 3) / 4; ++i) {
        const int pc = (wave + 4 * i) * 64 + lane;
        const int row = pc / 4, ph = pc % 4;
        vvoff[i] = (unsigned)(row * N + ((ph ^ vswz(row)) << 4));
    }
    auto issue = [&](int j, uint8_t *kd, uint8_t *vd) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < (KSEG + 3) / 4; ++i)
            if (wave + 4 * i < KSEG)
                buffer_to_lds16(krs, (bf16 *)(kd + (wave + 4 * i) * 1024), kvoff[i], j * BC * D);
#pragma unroll
        for (int i = 0; i < (VSEG + 3) / 4; ++i)
            if (wave + 4 * i < VSEG)
                buffer_to_lds16(vrs, (bf16 *)(vd + (wave + 4 * i) * 1024), vvoff[i], j * BC);
    };

    // this lane's rows / chunks in the tiles
    const int krow = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);   // permuted key row

    float m = -INFINITY, lsum = 0.f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        oacc[db] = f32x16{};

    auto compute = [&](auto masked, int j, const uint8_t *kt, const uint8_t *vt) __attribute__((always_inline)) {
        const int kbase = j * BC;
        if (CAUSAL && kbase > wq0 + 31)
            return;
        const float c_t = c_q * ksc[kbase >> 7];
        f32x16 s[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const int r = kc * 32 + krow;
            i32x8 ka[KSTEPS];
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                const int ch = 4 * st + 2 * hf;
                const u32x4 x0 = lds16(kt + r * D + ((ch ^ kswz<D>(r)) << 4));
                const u32x4 x1 = lds16(kt + r * D + (((ch + 1) ^ kswz<D>(r)) << 4));
                ka[st] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                               (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
            }
            __builtin_amdgcn_sched_barrier(0);
            s[kc] = f32x16{};
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st)
                s[kc] = mfma_fp8(ka[st], qreg[st], s[kc]);
        }
        if (decltype(masked)::value && ((kbase + BC > kv_len) || (CAUSAL && kbase + BC - 1 > wq0))) {
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kbase + kc * 32 + 16 * hf + i;
                    if (key >= kv_len || (CAUSAL && key > qrow))
                        s[kc][i] = -INFINITY;
                }
        }
        // probabilities: fp32 row sum, E4M3 operand bytes (slot 16 kc + i)
        int pw[8];
        auto probs = [&](float m_ref) __attribute__((always_inline)) -> float {
            float acc = 0.f;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int i = 0; i < 16; i += 4) {
                    float pv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pv[e] = exp2_hw(fmaf(s[kc][i + e], c_t, -m_ref));
                        acc += pv[e];
                    }
                    int wd = 0;
                    wd = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], wd, false);
                    wd = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], wd, true);
                    pw[(16 * kc + i) / 4] = wd;
                }
            return acc;
        };
        // Against the current reference first: every probability is at most
        // the lane's partial row sum, so while no partial sum passes 2^TAU
        // the lazy rule would not move the reference and the tile maximum is
        // not needed (same result as taking it first).
        float rs = 0.f;
        bool slow = __any(m == -INFINITY);
        if (!slow) {
            rs = probs(m);
            slow = __any(!(rs <= kPassLimit8));   // also catches inf
        }
        if (slow) {
            float mx = -INFINITY;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    mx = fmaxf(mx, s[kc][i]);
            const float mt = pair_max(mx) * c_t;
            if (__any(mt > m + TAU8)) {
                const float m_new = fmaxf(m, mt);
                const float alpha = exp2_hw(m - m_new);
                m = m_new;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    oacc[db] *= alpha;
            }
            rs = probs((m == -INFINITY) ? 0.f : m);
        }
        lsum += rs;
        const i32x8 pop = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
        // O^T += V^T P^T
        i32x8 va[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int r = db * 32 + l32;
            const u32x4 x0 = lds16(vt + r * BC + ((hf ^ vswz(r)) << 4));
            const u32x4 x1 = lds16(vt + r * BC + (((2 + hf) ^ vswz(r)) << 4));
            va[db] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                           (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            oacc[db] = mfma_fp8(va[db], pop, oacc[db]);
    };

    auto step = [&](auto masked, int t) __attribute__((always_inline)) {
        if (t + 1 < n_tiles)
            issue(t + 1, k1s, v1s);
        compute(masked, t, k0s, v0s);
        wait_vmem();
        __syncthreads();
        if (t + 1 < n_tiles) {
            if (t + 2 < n_tiles)
                issue(t + 2, k0s, v0s);
            compute(masked, t + 1, k1s, v1s);
            wait_vmem();
            __syncthreads();
        }
    };
    int n_plain = min(n_tiles, kv_len / BC);
    if (CAUSAL)
        n_plain = min(n_plain, (q0 + 1) / BC);
    const int t_mask = n_plain & ~1;
    if (n_tiles > 0)
        issue(0, k0s, v0s);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < t_mask; t += 2)
        step(std::false_type{}, t);
    for (int t = t_mask; t < n_tiles; t += 2)
        step(std::true_type{}, t);

    const float ltot = pair_sum(lsum);
    const float inv = ltot > 0.f ? p.vs[bh] / ltot : 0.f;
    if (qrow < N) {
        bf16 *O = p.o + (size_t)bh * N * D + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ov[e] = (bf16)(oacc[db][4 * g + e] * inv);
                *(bf16x4 *)(O + db * 32 + 8 * g + 4 * hf) = ov;
            }
        if (hf == 0)
            p.lse[(size_t)bh * N + qrow] = ltot > 0.f ? kLn2 * (m + __log2f(ltot)) : -INFINITY;
    }
}

template <int D, bool ROT>
hipError_t launch_quant_d(QuantArgs a, bool per_head, bool transpose, hipStream_t s)
{
    const dim3 grid((unsigned)(a.B * a.H * a.nblk)), block(256);
    if (per_head) {
        quant_amax_kernel<D, ROT><<<grid, block, 0, s>>>(a);
        if (transpose)
            quant_kernel<D, ROT, true, true><<<grid, block, 0, s>>>(a);
        else
            quant_kernel<D, ROT, true, false><<<grid, block, 0, s>>>(a);
    } else {
        if (transpose)
            quant_kernel<D, ROT, false, true><<<grid, block, 0, s>>>(a);
        else
            quant_kernel<D, ROT, false, false><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_fwd_fp8(const void *q8, const void *k8, const void *v8t, const float *qs,
                          const float *ks, const float *vs, void *o, float *lse, int B, int H,
                          int N, int d, bool causal, float scale, const int32_t *kv_lens,
                          hipStream_t s)
{
    Fp8FwdArgs a{(const uint8_t *)q8, (const uint8_t *)k8, (const uint8_t *)v8t, qs, ks, vs,
                 (bf16 *)o, lse, B, H, N, (N + 127) / 128, scale * kLog2e, kv_lens};
    const dim3 grid((unsigned)(B * H * ((N + 127) / 128))), block(256);
    if (d == 64) {
        if (causal)
            fwd_fp8_kernel<64, true><<<grid, block, 0, s>>>(a);
        else
            fwd_fp8_kernel<64, false><<<grid, block, 0, s>>>(a);
    } else {
        if (causal)
            fwd_fp8_kernel<128, true><<<grid, block, 0, s>>>(a);
        else
            fwd_fp8_kernel<128, false><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_quant_fp8(const void *x, void *x8, float *descale, float *amax_ws,
                            const float *signs, int B, int H, int N, int d, bool per_head,
                            bool transpose, hipStream_t s)
{
    QuantArgs a{(const bf16 *)x, (uint8_t *)x8, descale, amax_ws, signs,
                (float)(1.0 / sqrt((double)d)), B, H, N, (N + 127) / 128};
    const bool rot = signs != nullptr;
    if (d == 64)
        return rot ? launch_quant_d<64, true>(a, per_head, transpose, s)
                   : launch_quant_d<64, false>(a, per_head, transpose, s);
    return rot ? launch_quant_d<128, true>(a, per_head, transpose, s)
               : launch_quant_d<128, false>(a, per_head, transpose, s);
}

} // namespace fa
