// fa_fwd.hip -- forward attention kernels for gfx950 (CDNA4).
//
// Exact attention O = softmax(scale Q K^T) V computed tile by tile with the
// running-statistics recurrence ("The Attention Matrix You Never Write Down",
// section "The running-statistics trick", steps 1-4; "FlashAttention:
// Mathematical Foundations, IO-Aware Tiling, Online Softmax, and Recomputation
// Dynamics", sections "Incremental Online Updates" and "IO-Aware Tiling
// Algorithm").  Per query row the kernel keeps the running maximum m, the
// running sum l and an unnormalised output accumulator; a new key tile with a
// larger maximum rescales l and the accumulator by exp(m - m'), and the
// accumulator is divided by l once at the end.  Only O and the row's
// log-sum-exp are written.
//
// Schedule.  One workgroup of 4 wave64s owns 128 query rows of one (b, h) and
// streams every key/value tile through LDS (queries outer, keys inner: the
// work partitioning of the same article's "FlashAttention-2" section, rather
// than the key-outer loop of its Algorithm 1, so O, m and l never leave
// registers).  Each wave owns 32 query rows.
//
// Data layout on chip.  The score tile is computed transposed, S^T = K Q^T,
// with v_mfma_f32_32x32x16_bf16: the MFMA result gives each lane one query
// column and 16 key rows, so the row max and row sum of a query are a
// reduction over the lane's own registers plus one exchange with the lane 32
// away.  The probabilities then feed O^T += V^T P^T directly as the B operand
// (same lane = same query, same key order), so P never touches LDS.
//
// Exponentials use exp2 with the scale folded in: t = S * scale * log2(e),
// P = 2^(t - m) with m tracked in log2 units, and LSE = ln2 * (m + log2 l).
//
// Lazy rescaling.  The reference maximum m a row's exponentials are taken
// against only moves when a tile's maximum exceeds it by more than TAU = 8
// (log2 units); otherwise the tile's exponentials are taken against the old
// m and may reach 2^8.  The result is unchanged: l and the accumulator share
// the same reference, and the final division cancels it.  This skips the
// O(d) rescale of the accumulator on most tiles.  Since every exponential
// taken against m is at most the row's partial sum, the tile maximum itself
// is only computed when that sum passes 2^TAU: most tiles skip the max
// reduction and give the same result.
//
// Tiles in LDS: K and V are both row-major and swizzled (fa_tile.h), copied
// from HBM by direct buffer->LDS loads.  K is read as the A operand of
// S^T = K Q^T one 16-byte chunk per lane; V^T, the A operand of
// O^T += V^T P^T, comes straight from the row-major V tile through the
// hardware transpose read.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {

constexpr float TAU = 8.f;             // lazy-rescale threshold (log2 units)
constexpr float kPassLimit = 256.f;    // 2^TAU

// Workgroup barrier that waits for this wave's LDS reads but leaves its
// buffer->LDS copies in flight (the plain barrier would wait for those too).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// wait until at most N vector-memory loads of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_but()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------------------
// bf16 forward.  D = head dim, BC = keys per tile, BR = 128 queries per
// workgroup.  SPARSE walks the nonzero 128-blocks of the workgroup's mask row.
//
// Tiles reach LDS by direct buffer->LDS loads into two stages (the loop is
// unrolled by two so the stage of each access is known at compile time); K
// and V stages are refilled separately, as soon as the phase reading them is
// done, two tiles ahead.
//
// D = 256 keeps the same schedule: Q's operands (64 registers) and the O^T
// accumulator (128) need the 512-register budget of one wave per SIMD, and
// two stages of 64-key K and V tiles take 128 KB of the 160 KB LDS.
template <int D, int BC, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, D == 256 ? 1 : 2) void fwd_bf16_kernel(FwdArgs p, float c_log2)
{
    constexpr int BR = 128;
    constexpr int KSTEPS = D / 16;         // k-steps of S^T over d
    constexpr int NKC = BC / 32;           // 32-key chunks per tile
    constexpr int NDB = D / 32;            // 32-wide d blocks of O^T

    __shared__ __attribute__((aligned(1024))) bf16 k0s[BC * D];
    __shared__ __attribute__((aligned(1024))) bf16 v0s[BC * D];
    __shared__ __attribute__((aligned(1024))) bf16 k1s[BC * D];
    __shared__ __attribute__((aligned(1024))) bf16 v1s[BC * D];
    __shared__ int blist[SPARSE ? MAX_MASK_BLOCKS : 1];
    __shared__ int bcount;

    const int N = p.N;
    const int n_qblk = (N + BR - 1) / BR;
    const int total = p.B * p.H * n_qblk;
    int bh, qb;
    if (CAUSAL) {
        const int grp = l2_group(N, 4 * D);
        causal_item(blockIdx.x, p.B * p.H, n_qblk, grp, bh, qb);
        // rank 0 = the last block (longest rows), after the rotation that
        // starts the ranks past the first round of workgroups first
        const int rot = causal_rotation(p.B * p.H, n_qblk, grp, p.wg_slots);
        qb = n_qblk - 1 - (qb + n_qblk - rot) % n_qblk;
    } else {
        const int w = xcd_remap(blockIdx.x, total);
        bh = w / n_qblk;
        qb = w % n_qblk;
    }
    const int b = bh / p.H;

    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = tid & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int q0 = qb * BR;
    const int wq0 = q0 + wave * 32;          // first query of this wave
    const int qrow = wq0 + l32;              // this lane's query

    const size_t head_off = (size_t)bh * N * D;
    const bf16 *Q = (const bf16 *)p.q + head_off;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc((const bf16 *)p.k + head_off, N, D);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc((const bf16 *)p.v + head_off, N, D);

    int kv_len = N;
    if (p.kv_lens) {
        kv_len = p.kv_lens[b];
        kv_len = kv_len < 0 ? 0 : (kv_len > N ? N : kv_len);
    }

    // ---- the tiles this workgroup visits
    int n_tiles;
    constexpr int TPB = 128 / BC;            // tiles per 128-block (sparse)
    if constexpr (SPARSE) {
        if (wave == 0)
            list_nonzero(p.mask + (size_t)qb * p.nb, p.nb, 1, blist, &bcount);
        __syncthreads();
        n_tiles = __builtin_amdgcn_readfirstlane(bcount) * TPB;
    } else {
        int kv_end = kv_len;
        if (CAUSAL)
            kv_end = min(kv_end, q0 + BR);
        n_tiles = (kv_end + BC - 1) / BC;
    }
    auto tile_of = [&](int t) __attribute__((always_inline)) -> int {
        if constexpr (SPARSE)
            return __builtin_amdgcn_readfirstlane(blist[t / TPB]) * TPB + t % TPB;
        else
            return t;
    };

    // ---- Q as the B operand of S^T = K Q^T: lane holds its query's d-slice
    bf16x8 qreg[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        if (qrow < N)
            qreg[s] = *(const bf16x8 *)(Q + (size_t)qrow * D + s * 16 + hf * 8);
        else
            qreg[s] = bf16x8{};
    }

    using Dma = TileDma<BC, D, 4>;
    Dma dma;
    dma.init(wave);

    float m = -INFINITY;   // reference max (log2 units), same in both lane halves
    float lsum = 0.f;      // running sum, partial over this lane half's keys
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        oacc[db] = f32x16{};

    f32x16 s[NKC];         // S^T of the current tile, between its two phases

    // phase 1 of tile j: S^T = K_j Q^T
    auto compute_s = [&](int j, const bf16 *kt) __attribute__((always_inline)) {
        // whole tile above this wave's diagonal: nothing to add
        if (CAUSAL && j * BC > wq0 + 31)
            return;
        // operands first, then the products (keeps LDS latency off each MFMA)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            bf16x8 ka[KSTEPS];
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st)
                ka[st] = ld_row8<D>(kt, kc * 32 + l32, st * 16 + hf * 8);
            __builtin_amdgcn_sched_barrier(0);
            s[kc] = f32x16{};
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st)
                s[kc] = mfma_bf16(ka[st], qreg[st], s[kc]);
        }
    };
    // phase 2 of tile j: masks, softmax, O^T += V_j^T P^T.  MASKED instances
    // handle the trailing tiles that cross the causal diagonal or the key
    // length; the main loop runs the unmasked instance.
    auto compute_pv = [&](auto masked, int j, const bf16 *vt) __attribute__((always_inline)) {
        const int kbase = j * BC;
        if (CAUSAL && kbase > wq0 + 31)
            return;
        if (decltype(masked)::value && ((kbase + BC > kv_len) || (CAUSAL && kbase + BC - 1 > wq0))) {
            // register (kc, i) holds key kbase + 4 hf + o, o = 32 kc + 8 (i / 4) + i % 4: it is
            // allowed iff o <= lim (below the key length and, causal, not after the query),
            // one compare against a constant per score
            int lim = kv_len - 1 - kbase - 4 * hf;
            if (CAUSAL)
                lim = min(lim, qrow - kbase - 4 * hf);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kc * 32 + 8 * (i / 4) + (i % 4) > lim)
                        s[kc][i] = -INFINITY;
        }
        // Probabilities against the current reference m, with fp32 row sums
        // and bf16 operands for P V.  The reference must move (lazily: only
        // when the tile's maximum exceeds it by more than TAU) exactly when
        // some probability would pass 2^TAU, and every probability is at
        // most the lane's row sum, so the tile maximum is needed only when a
        // partial row sum passes 2^TAU (or the row has no reference yet):
        // the common tile skips the max reduction.  Either way the result is
        // the one the max-first order gives.
        // (the row sum starts at the first probability: an add to 0.0f is an
        // instruction, kept for -0, which an exponential never is)
        float rs = 0.f;
        bf16x8 pb[NKC][2];
        bool slow = __any(m == -INFINITY);
        if (!slow) {
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = exp2_hw(fmaf(s[kc][i], c_log2, -m));
                    rs = (kc == 0 && i == 0) ? pv : rs + pv;
                    pb[kc][i / 8][i % 8] = (bf16)pv;
                }
            slow = __any(!(rs <= kPassLimit));   // also catches inf
        }
        if (slow) {
            float mx = -INFINITY;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    mx = fmaxf(mx, s[kc][i]);
            const float mt = pair_max(mx) * c_log2;
            if (__any(mt > m + TAU)) {
                const float m_new = fmaxf(m, mt);
                const float alpha = exp2_hw(m - m_new);   // 0 when m = -inf
                m = m_new;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    oacc[db] *= alpha;
            }
            const float m_use = (m == -INFINITY) ? 0.f : m;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = exp2_hw(fmaf(s[kc][i], c_log2, -m_use));
                    rs = (kc == 0 && i == 0) ? pv : rs + pv;
                    pb[kc][i / 8][i % 8] = (bf16)pv;
                }
        }
        lsum += rs;
        // O^T += V_j^T P^T
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            bf16x8 va[NKC][2];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    va[kc][hh] = ld_tr8<D>(vt, kc * 32 + hh * 16, db * 32);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    oacc[db] = mfma_bf16(va[kc][hh], pb[kc][hh], oacc[db]);
        }
    };

    // Tile t (LDS stage ST = t & 1) in two phases separated by a barrier, so
    // that K and V stages free up at different times: K_{t+2} is copied into
    // K_t's stage once every wave has finished S_t (barrier A), and V_{t+2}
    // into V_t's stage once every wave has finished P V (barrier B).  Each
    // copy then has about one and a half tiles of compute to land before its
    // wait, which lets the two copies issued since stay in flight.  Every
    // tile issues both copies (past the last tile, duplicates of it into a
    // free stage), so the in-flight count is fixed.
    constexpr int kCopies = 2 * Dma::PER_WAVE;  // loads of the two newest copies
    auto tile = [&](auto masked, int t, auto st_c) __attribute__((always_inline)) {
        constexpr int ST = decltype(st_c)::value;
        bf16 *kt = ST ? k1s : k0s;
        bf16 *vt = ST ? v1s : v0s;
        const int j = tile_of(t);
        const int j2 = tile_of(min(t + 2, n_tiles - 1));
        compute_s(j, kt);
        wait_vmem_but<kCopies>();                // V_t has landed
        lds_barrier();                           // A
        dma.issue(krs, j2 * BC, kt, wave);
        compute_pv(masked, j, vt);
        wait_vmem_but<kCopies>();                // K_{t+1} has landed
        lds_barrier();                           // B
        dma.issue(vrs, j2 * BC, vt, wave);
    };
    // leading tiles that no wave needs to mask: whole tiles below the key
    // length and (causal) entirely at or left of the block's first query
    int n_plain = n_tiles;
    if constexpr (!SPARSE) {
        n_plain = min(n_tiles, kv_len / BC);
        if (CAUSAL)
            n_plain = min(n_plain, (q0 + 1) / BC);
    }
    const int t_mask = n_plain & ~1;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if (n_tiles > 0) {
        const int j1 = tile_of(min(1, n_tiles - 1));
        dma.issue(krs, tile_of(0) * BC, k0s, wave);
        dma.issue(vrs, tile_of(0) * BC, v0s, wave);
        dma.issue(krs, j1 * BC, k1s, wave);
        dma.issue(vrs, j1 * BC, v1s, wave);
    }
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < t_mask; t += 2) {
        tile(std::false_type{}, t, I0{});
        tile(std::false_type{}, t + 1, I1{});
    }
    for (int t = t_mask; t < n_tiles; t += 2) {
        tile(std::true_type{}, t, I0{});
        if (t + 1 < n_tiles)
            tile(std::true_type{}, t + 1, I1{});
    }
    wait_vmem();

    // ---- epilogue: O = acc / l, LSE = ln2 (m + log2 l)
    const float ltot = pair_sum(lsum);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (qrow < N) {
        bf16 *O = (bf16 *)p.o + head_off + (size_t)qrow * D;
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

// ---------------------------------------------------------------------------
// fp32 forward (full-precision operands through v_mfma_f32_32x32x2_f32).
// Same transposed schedule; 32 keys per tile; one LDS buffer.  With one
// element of k per lane the V operand is a plain row-major read.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(FwdArgs p, float c_log2)
{
    constexpr int BR = 128, BC = 32;
    constexpr int KSTEPS = D / 2;
    constexpr int NDB = D / 32;
    constexpr int KS = D + 1;   // K row stride (floats)
    constexpr int VS = D + 4;   // V row stride (floats)
    __shared__ float ks[BC * KS];
    __shared__ float vs[BC * VS];

    const int N = p.N;
    const int n_qblk = (N + BR - 1) / BR;
    const int total = p.B * p.H * n_qblk;
    int bh, qb;
    if (CAUSAL) {
        causal_item(blockIdx.x, p.B * p.H, n_qblk, l2_group(N, 8 * D), bh, qb);
        qb = n_qblk - 1 - qb;                // rank 0 = the last block: longest rows
    } else {
        const int w = xcd_remap(blockIdx.x, total);
        bh = w / n_qblk;
        qb = w % n_qblk;
    }
    const int b = bh / p.H;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int q0 = qb * BR;
    const int wq0 = q0 + wave * 32;
    const int qrow = wq0 + l32;
    const size_t head_off = (size_t)bh * N * D;
    const float *Q = (const float *)p.q + head_off;
    const float *K = (const float *)p.k + head_off;
    const float *V = (const float *)p.v + head_off;

    int kv_len = N;
    if (p.kv_lens) {
        kv_len = p.kv_lens[b];
        kv_len = kv_len < 0 ? 0 : (kv_len > N ? N : kv_len);
    }
    int kv_end = kv_len;
    if (CAUSAL)
        kv_end = min(kv_end, q0 + BR);
    const int n_tiles = (kv_end + BC - 1) / BC;

    float qreg[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
        qreg[s] = qrow < N ? Q[(size_t)qrow * D + 2 * s + hf] : 0.f;

    float m = -INFINITY, lsum = 0.f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        oacc[db] = f32x16{};

    for (int t = 0; t < n_tiles; ++t) {
        const int kbase = t * BC;
        for (int idx = tid; idx < BC * D; idx += 256) {
            const int row = idx / D, col = idx % D;
            const int key = kbase + row;
            ks[row * KS + col] = key < N ? K[(size_t)key * D + col] : 0.f;
            vs[row * VS + col] = key < N ? V[(size_t)key * D + col] : 0.f;
        }
        __syncthreads();
        const bool skip = CAUSAL && kbase > wq0 + 31;
        if (!skip) {
            f32x16 s = f32x16{};
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st)
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[l32 * KS + 2 * st + hf], qreg[st], s, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kbase + 8 * (i / 4) + 4 * hf + (i % 4);
                if (key >= kv_len || (CAUSAL && key > qrow))
                    s[i] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                mx = fmaxf(mx, s[i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m, mx * c_log2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2_hw(m - m_use);
            m = m_new;
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[i] = exp2_hw(fmaf(s[i], c_log2, -m_use));
                rs += s[i];
            }
            lsum = alpha * lsum + rs;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                oacc[db] *= alpha;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 8 * (i / 4) + 4 * hf + (i % 4);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * VS + db * 32 + l32], s[i],
                                                                   oacc[db], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (qrow < N) {
        float *O = (float *)p.o + head_off + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                O[db * 32 + 8 * (i / 4) + 4 * hf + (i % 4)] = oacc[db][i] * inv;
        if (hf == 0)
            p.lse[(size_t)bh * N + qrow] = ltot > 0.f ? kLn2 * (m + __log2f(ltot)) : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// bf16 forward with 256-key tiles: the block-size end of the key-tile sweep
// (the pages report fewer HBM accesses and less run time for larger blocks
// up to about 256, "Attention" chapter of learn-kernels.com, paragraph on
// the block-size sweep).  One LDS stage holds the whole K and V tile (128 KB
// at d = 128, 64 KB at d = 64), so one workgroup of 4 waves runs per CU and
// a tile's copy cannot overlap the previous tile's work: copy, barrier, the
// tile's eight 32-key chunks (S, masks, softmax, P V each, as in
// fwd_bf16_kernel), barrier.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_bf16_t256_kernel(FwdArgs p, float c_log2)
{
    constexpr int BR = 128, BC = 256;
    constexpr int KSTEPS = D / 16;
    constexpr int NDB = D / 32;
    constexpr int NCH = BC / 32;            // 32-key chunks per tile

    __shared__ __attribute__((aligned(1024))) bf16 ks[BC * D];
    __shared__ __attribute__((aligned(1024))) bf16 vs[BC * D];

    const int N = p.N;
    const int n_qblk = (N + BR - 1) / BR;
    const int total = p.B * p.H * n_qblk;
    int bh, qb;
    if (CAUSAL) {
        causal_item(blockIdx.x, p.B * p.H, n_qblk, l2_group(N, 4 * D), bh, qb);
        qb = n_qblk - 1 - qb;                // rank 0 = the last block: longest rows
    } else {
        const int w = xcd_remap(blockIdx.x, total);
        bh = w / n_qblk;
        qb = w % n_qblk;
    }
    const int b = bh / p.H;
    const int tid = threadIdx.x;
    const int wave = wave_id(), lane = tid & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int q0 = qb * BR;
    const int wq0 = q0 + wave * 32;
    const int qrow = wq0 + l32;

    const size_t head_off = (size_t)bh * N * D;
    const bf16 *Q = (const bf16 *)p.q + head_off;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc((const bf16 *)p.k + head_off, N, D);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc((const bf16 *)p.v + head_off, N, D);

    int kv_len = N;
    if (p.kv_lens) {
        kv_len = p.kv_lens[b];
        kv_len = kv_len < 0 ? 0 : (kv_len > N ? N : kv_len);
    }
    int kv_end = kv_len;
    if (CAUSAL)
        kv_end = min(kv_end, q0 + BR);
    const int n_tiles = (kv_end + BC - 1) / BC;

    bf16x8 qreg[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
        qreg[s] = qrow < N ? *(const bf16x8 *)(Q + (size_t)qrow * D + s * 16 + hf * 8) : bf16x8{};

    using Dma = TileDma<BC, D, 4>;
    Dma dma;
    dma.init(wave);

    float m = -INFINITY, lsum = 0.f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        oacc[db] = f32x16{};

    for (int t = 0; t < n_tiles; ++t) {
        dma.issue(krs, t * BC, ks, wave);
        dma.issue(vrs, t * BC, vs, wave);
        wait_vmem();
        __syncthreads();
        for (int c = 0; c < NCH; ++c) {
            const int kbase = t * BC + c * 32;
            if (kbase >= kv_end || (CAUSAL && kbase > wq0 + 31))
                break;                       // chunks only grow from here (wave-uniform)
            f32x16 s = f32x16{};
            bf16x8 ka[KSTEPS];
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st)
                ka[st] = ld_row8<D>(ks, c * 32 + l32, st * 16 + hf * 8);
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st)
                s = mfma_bf16(ka[st], qreg[st], s);
            if (kbase + 32 > kv_len || (CAUSAL && kbase + 31 > wq0)) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kbase + 8 * (i / 4) + 4 * hf + (i % 4);
                    if (key >= kv_len || (CAUSAL && key > qrow))
                        s[i] = -INFINITY;
                }
            }
            // running maximum moved lazily (threshold TAU), as in fwd_bf16_kernel
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                mx = fmaxf(mx, s[i]);
            const float mt = pair_max(mx) * c_log2;
            if (__any(mt > m + TAU)) {
                const float m_new = fmaxf(m, mt);
                const float alpha = exp2_hw(m - m_new);
                m = m_new;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    oacc[db] *= alpha;
            }
            const float m_use = (m == -INFINITY) ? 0.f : m;
            bf16x8 pb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = exp2_hw(fmaf(s[i], c_log2, -m_use));
                lsum += pv;
                pb[i / 8][i % 8] = (bf16)pv;
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 v0 = ld_tr8<D>(vs, c * 32, db * 32);
                const bf16x8 v1 = ld_tr8<D>(vs, c * 32 + 16, db * 32);
                oacc[db] = mfma_bf16(v0, pb[0], oacc[db]);
                oacc[db] = mfma_bf16(v1, pb[1], oacc[db]);
            }
        }
        __syncthreads();                     // every wave done with this tile
    }

    const float ltot = pair_sum(lsum);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (qrow < N) {
        bf16 *O = (bf16 *)p.o + head_off + (size_t)qrow * D;
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

template <int D, bool CAUSAL>
static hipError_t launch_t256_inst(const FwdArgs &a, hipStream_t s)
{
    const int n_qblk = (a.N + 127) / 128;
    FwdArgs args = a;
    float c = a.scale * kLog2e;
    void *kargs[] = {&args, &c};
    return hipLaunchKernel((const void *)&fwd_bf16_t256_kernel<D, CAUSAL>, dim3(a.B * a.H * n_qblk),
                           dim3(256), kargs, 0, s);
}

// ---------------------------------------------------------------------------
// workgroups of a kernel resident at once on one XCD (0 if unknown), queried
// once per kernel: the number of CUs per XCD times the kernel's occupancy
static int xcd_slots(const void *fn, int block)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0) != hipSuccess)
        return 0;
    return cus % 8 == 0 ? cus / 8 * per_cu : 0;
}

template <int D, int BC, bool CAUSAL, bool SPARSE>
static hipError_t launch_bf16_inst(const FwdArgs &a, hipStream_t s)
{
    const int n_qblk = (a.N + 127) / 128;
    const dim3 grid(a.B * a.H * n_qblk), block(256);
    FwdArgs args = a;
    if constexpr (CAUSAL) {
        static const int slots = xcd_slots((const void *)&fwd_bf16_kernel<D, BC, CAUSAL, SPARSE>, 256);
        args.wg_slots = slots;
    }
    float c = a.scale * kLog2e;
    void *kargs[] = {&args, &c};
    return hipLaunchKernel((const void *)&fwd_bf16_kernel<D, BC, CAUSAL, SPARSE>, grid, block,
                           kargs, 0, s);
}

template <int D, int BC>
static hipError_t launch_bf16_d_bc(const FwdArgs &a, bool causal, bool sparse, hipStream_t s)
{
    if (sparse)
        return launch_bf16_inst<D, BC, false, true>(a, s);
    return causal ? launch_bf16_inst<D, BC, true, false>(a, s)
                  : launch_bf16_inst<D, BC, false, false>(a, s);
}

hipError_t launch_fwd_bf16(const FwdArgs &a, int d, int tile_n, bool causal, bool sparse,
                           hipStream_t s)
{
    if (tile_n == 0)
        tile_n = 64;
    if (d == 64 && tile_n == 64)
        return launch_bf16_d_bc<64, 64>(a, causal, sparse, s);
    if (d == 64 && tile_n == 128)
        return launch_bf16_d_bc<64, 128>(a, causal, sparse, s);
    if (d == 128 && tile_n == 64)
        return launch_bf16_d_bc<128, 64>(a, causal, sparse, s);
    if (d == 128 && tile_n == 128)
        return launch_bf16_d_bc<128, 128>(a, causal, sparse, s);
    if (d == 256 && tile_n == 64)
        return launch_bf16_d_bc<256, 64>(a, causal, sparse, s);
    if (tile_n == 256 && !sparse && (d == 64 || d == 128)) {
        if (d == 64)
            return causal ? launch_t256_inst<64, true>(a, s) : launch_t256_inst<64, false>(a, s);
        return causal ? launch_t256_inst<128, true>(a, s) : launch_t256_inst<128, false>(a, s);
    }
    if (d == 256 && tile_n == 32)
        return launch_bf16_d_bc<256, 32>(a, causal, sparse, s);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_f32(const FwdArgs &a, int d, bool causal, hipStream_t s)
{
    const int n_qblk = (a.N + 127) / 128;
    const dim3 grid(a.B * a.H * n_qblk), block(256);
    FwdArgs args = a;
    float c = a.scale * kLog2e;
    void *kargs[] = {&args, &c};
    const void *fn;
    if (d == 64)
        fn = causal ? (const void *)&fwd_f32_kernel<64, true> : (const void *)&fwd_f32_kernel<64, false>;
    else if (d == 128)
        fn = causal ? (const void *)&fwd_f32_kernel<128, true> : (const void *)&fwd_f32_kernel<128, false>;
    else
        return hipErrorInvalidValue;
    return hipLaunchKernel(fn, grid, block, kargs, 0, s);
}

} // namespace fa
