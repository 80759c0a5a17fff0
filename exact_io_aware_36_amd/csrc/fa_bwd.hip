// fa_bwd.hip -- backward attention kernels for gfx950 (CDNA4).
//
// The forward pass kept only O and the row log-sum-exp; the backward pass
// rebuilds each score tile S_ij and probability tile P_ij on chip from Q, K
// and that statistic instead of reading a stored N x N matrix
// ("FlashAttention: Mathematical Foundations, IO-Aware Tiling, Online Softmax,
// and Recomputation Dynamics", section "Backward Pass and Activation
// Recomputation"; "The Attention Matrix You Never Write Down", section
// "Tiling forward, recomputing backward").  With the stored LSE the
// probabilities need no max pass: P = exp(scale S - LSE).  The gradient
// formulas are the chain rule of O = softmax(scale Q K^T) V with the loss
// sum(O * dO): dV = P^T dO, dP = dO V^T, D_i = dO_i . O_i,
// dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
//
// Three launches on one stream:
//   1. bwd_dot_kernel: D_i = dO_i . O_i (fp32) and LSE_i * log2(e) into the
//      workspace.
//   2. bwd_dkdv_kernel: keys outer.  A workgroup owns 128 keys of one
//      (b, h) (32 per wave, held in registers as MFMA operands) and walks the
//      query tiles, accumulating dK and dV in registers.
//   3. bwd_dq_kernel: queries outer.  A workgroup owns 128 queries and walks
//      the key tiles, accumulating dQ in registers.
// Block-sparse instances walk only the nonzero blocks of the mask: the
// dK/dV workgroup's 128 keys are one mask column block (it visits the query
// tiles of that column's nonzero row blocks), the dQ workgroup's 128 queries
// one mask row block (the key tiles of that row's nonzero column blocks).
// No atomics: every output element is written by exactly one lane, so the
// result is deterministic.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16).  In the key-outer kernel the
// score tile is S (queries x keys), so each lane holds one key and 16 query
// rows; P and dS then feed dV^T += dO^T P and dK^T += Q^T dS as B operands
// without leaving registers, and the A operands dO^T, Q^T come from the
// row-major Q and dO tiles through the hardware transpose read.  In the
// query-outer kernel the tile is S^T, each lane holds one query (so LSE_i and
// D_i are lane-local), and dQ^T += K^T dS^T reads K^T from the row-major K
// tile the same way.  Tiles are swizzled and double-buffered (fa_tile.h).
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {

namespace {

// D_i = dO_i . O_i in fp32, and the row's LSE in log2 units ----------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const bf16 *__restrict__ o,
                                                      const bf16 *__restrict__ dout,
                                                      const float *__restrict__ lse,
                                                      float *__restrict__ dvec,
                                                      float *__restrict__ lse2, int rows)
{
    constexpr int CPR = D / 8;             // threads per row
    constexpr int RPB = 256 / CPR;         // rows per block
    const int r = blockIdx.x * RPB + threadIdx.x / CPR;
    const int c = (threadIdx.x % CPR) * 8;
    float acc = 0.f;
    if (r < rows) {
        const bf16x8 a = *(const bf16x8 *)(o + (size_t)r * D + c);
        const bf16x8 g = *(const bf16x8 *)(dout + (size_t)r * D + c);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc = fmaf((float)a[e], (float)g[e], acc);
    }
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off);
    if (r < rows && threadIdx.x % CPR == 0) {
        dvec[r] = acc;
        const float l = lse[r];
        lse2[r] = (l == -INFINITY) ? INFINITY : l * kLog2e;   // a row with no key: P = 0
    }
}

// dK, dV: keys outer ------------------------------------------------------
// Q and dO tiles (and their rows' LSE and D) reach LDS by direct buffer->LDS
// loads into two stages; the loop is unrolled by two.  Query rows past N read
// as zeros (Q, dO, LSE, D all 0), which makes their dS and P^T dO terms 0.
//
// MODE 0 computes dK and dV together.  At d = 256 the K, V operands and the
// two accumulators of a wave's 32 keys do not fit one wave's registers, so
// the work is split over two launches: MODE 1 (dV only: S, P, dV^T += dO^T P)
// and MODE 2 (dK only: S, dP, dS, dK^T += Q^T dS), recomputing S once more.
template <int D, bool CAUSAL, bool SPARSE, int MODE>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(BwdArgs p, float c_log2)
{
    constexpr bool DO_DV = MODE != 2, DO_DK = MODE != 1;
    constexpr int BKV = 128, BQ = 64;
    constexpr int KSTEPS = D / 16;
    constexpr int NQC = BQ / 32;           // 32-query chunks per tile
    constexpr int NDB = D / 32;
    constexpr int PF = D >= 128 ? 2 : KSTEPS;   // S, dP operands loaded ahead of their products

    __shared__ __attribute__((aligned(1024))) bf16 q0s[BQ * D];
    __shared__ __attribute__((aligned(1024))) bf16 g0s[BQ * D];
    __shared__ __attribute__((aligned(1024))) bf16 q1s[BQ * D];
    __shared__ __attribute__((aligned(1024))) bf16 g1s[BQ * D];
    __shared__ __attribute__((aligned(256))) float l0s[BQ];
    __shared__ __attribute__((aligned(256))) float d0s[BQ];
    __shared__ __attribute__((aligned(256))) float l1s[BQ];
    __shared__ __attribute__((aligned(256))) float d1s[BQ];

    const int N = p.N;
    const int n_kb = (N + BKV - 1) / BKV;
    const int total = p.B * p.H * n_kb;
    const int w = xcd_remap(blockIdx.x, total);
    const int bh = w / n_kb;
    const int kb = w % n_kb;               // causal: low key blocks have the most work
    const int b = bh / p.H;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int k0 = kb * BKV;
    const int wk0 = k0 + wave * 32;
    const int key = wk0 + l32;

    const size_t head_off = (size_t)bh * N * D;
    const bf16 *K = (const bf16 *)p.k + head_off;
    const bf16 *V = (const bf16 *)p.v + head_off;
    const __amdgpu_buffer_rsrc_t qrs = head_rsrc((const bf16 *)p.q + head_off, N, D);
    const __amdgpu_buffer_rsrc_t grs = head_rsrc((const bf16 *)p.dout + head_off, N, D);
    const __amdgpu_buffer_rsrc_t lrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(p.lse2 + (size_t)bh * N), (short)0, N * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t drs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(p.dvec + (size_t)bh * N), (short)0, N * 4, 0x00020000);

    int kv_len = N;
    if (p.kv_lens) {
        kv_len = p.kv_lens[b];
        kv_len = kv_len < 0 ? 0 : (kv_len > N ? N : kv_len);
    }

    // K and V of this lane's key as B operands (k = d)
    bf16x8 kreg[KSTEPS], vreg[KSTEPS];
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
        if (key < N) {
            kreg[st] = *(const bf16x8 *)(K + (size_t)key * D + st * 16 + hf * 8);
            vreg[st] = DO_DK ? *(const bf16x8 *)(V + (size_t)key * D + st * 16 + hf * 8) : bf16x8{};
        } else {
            kreg[st] = bf16x8{};
            vreg[st] = bf16x8{};
        }
    }

    f32x16 dk_acc[NDB], dv_acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dk_acc[db] = f32x16{};
        dv_acc[db] = f32x16{};
    }

    // the query tiles visited, in order: dense, all tiles from the diagonal
    // (causal) or from 0; block-sparse, the two tiles of every nonzero row
    // block of this key block's mask column
    __shared__ int blist[SPARSE ? MAX_MASK_BLOCKS : 1];
    __shared__ int bcount;
    const int n_qt = (N + BQ - 1) / BQ;
    const int qt_begin = (CAUSAL ? k0 / BQ : 0);
    int n_vis;
    if constexpr (SPARSE) {
        if (wave == 0)
            list_nonzero(p.mask + kb, p.nb, p.nb, blist, &bcount);
        __syncthreads();
        n_vis = __builtin_amdgcn_readfirstlane(bcount) * (128 / BQ);
    } else {
        n_vis = (k0 < kv_len) ? n_qt - qt_begin : 0;   // no allowed key: nothing to do
    }
    auto qtile = [&](int t) __attribute__((always_inline)) -> int {
        if constexpr (SPARSE)
            return __builtin_amdgcn_readfirstlane(blist[t / (128 / BQ)]) * (128 / BQ) + t % (128 / BQ);
        else
            return qt_begin + t;
    };
    const bool wave_live = wk0 < kv_len;

    TileDma<BQ, D, 4> dma;
    dma.init(wave);
    auto issue = [&](int it, bf16 *qd, bf16 *gd, float *ld, float *dd) __attribute__((always_inline)) {
        const int qbase = it * BQ;
        dma.issue(qrs, qbase, qd, wave);
        dma.issue(grs, qbase, gd, wave);
        if (wave == 0)
            buffer_to_lds4(lrs, ld, lane * 4, qbase * 4);
        else if (wave == 1 && DO_DK)
            buffer_to_lds4(drs, dd, lane * 4, qbase * 4);
    };

    // MASKED applies the causal mask.  Only the two query tiles that hold this
    // workgroup's diagonal (the first two visited, qbase = k0 and k0 + 64)
    // need it; they are peeled off the main loop below.  Key padding needs no
    // mask here: a padded key's P reaches only its own dK, dV row, which the
    // store writes as zero.
    auto compute = [&](auto masked, int it, const bf16 *qt, const bf16 *gt, const float *lt,
                       const float *dt) __attribute__((always_inline)) {
        const int qbase = it * BQ;
        if (!wave_live || (CAUSAL && qbase + BQ - 1 < wk0))
            return;
        const bool need_mask = decltype(masked)::value && qbase < wk0 + 31;
        // One 32-query chunk at a time: S, dP, then P and dS, then
        // dV^T += dO^T P and dK^T += Q^T dS.  The S, dP operands are read PF
        // k-steps ahead of their products (at d = 128 two steps, which keeps
        // the products' results out of the accumulation registers; at d = 64
        // all of them first), the group barriers fixing that order.
#pragma unroll
        for (int q0c = 0; q0c < NQC; ++q0c) {
            constexpr int G = 1;
            f32x16 s[G], dp[G];
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int qc = q0c + u;
                s[u] = f32x16{};
                dp[u] = f32x16{};
                bf16x8 qa[KSTEPS], ga[KSTEPS];
#pragma unroll
                for (int st = 0; st < PF; ++st) {
                    qa[st] = ld_row8<D>(qt, qc * 32 + l32, st * 16 + hf * 8);
                    if constexpr (DO_DK)
                        ga[st] = ld_row8<D>(gt, qc * 32 + l32, st * 16 + hf * 8);
                }
#pragma unroll
                for (int st = 0; st < KSTEPS; ++st) {
                    s[u] = mfma_bf16(qa[st], kreg[st], s[u]);
                    if constexpr (DO_DK)
                        dp[u] = mfma_bf16(ga[st], vreg[st], dp[u]);
                    if (st + PF < KSTEPS) {
                        qa[st + PF] = ld_row8<D>(qt, qc * 32 + l32, (st + PF) * 16 + hf * 8);
                        if constexpr (DO_DK)
                            ga[st + PF] = ld_row8<D>(gt, qc * 32 + l32, (st + PF) * 16 + hf * 8);
                    }
                }
                constexpr int RD = DO_DK ? 2 : 1;   // operand reads and products per k-step
                __builtin_amdgcn_sched_group_barrier(0x100, RD * PF, 0);         // DS reads
#pragma unroll
                for (int st = 0; st < KSTEPS; ++st) {
                    __builtin_amdgcn_sched_group_barrier(0x008, RD, 0);          // MFMA
                    if (st + PF < KSTEPS)
                        __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);      // DS reads
                }
            }
            bf16x8 pb[G][2], dsb[G][2];
#pragma unroll
            for (int u = 0; u < G; ++u)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int trow = (q0c + u) * 32 + 8 * g + 4 * hf;
                    const f32x4 l4 = *(const f32x4 *)&lt[trow];
                    const f32x4 d4 = DO_DK ? *(const f32x4 *)&dt[trow] : f32x4{};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * g + e;
                        float pv = exp2_hw(fmaf(s[u][i], c_log2, -l4[e]));
                        if (need_mask && key > qbase + trow + e)
                            pv = 0.f;
                        if constexpr (DO_DV)
                            pb[u][i / 8][i % 8] = (bf16)pv;
                        if constexpr (DO_DK)
                            dsb[u][i / 8][i % 8] = (bf16)(pv * (dp[u][i] - d4[e]));
                    }
                }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                bf16x8 ga[G][2], qa[G][2];
#pragma unroll
                for (int u = 0; u < G; ++u)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        if constexpr (DO_DV)
                            ga[u][hh] = ld_tr8<D>(gt, (q0c + u) * 32 + hh * 16, db * 32);
                        if constexpr (DO_DK)
                            qa[u][hh] = ld_tr8<D>(qt, (q0c + u) * 32 + hh * 16, db * 32);
                    }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < G; ++u)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        if constexpr (DO_DV)
                            dv_acc[db] = mfma_bf16(ga[u][hh], pb[u][hh], dv_acc[db]);
                        if constexpr (DO_DK)
                            dk_acc[db] = mfma_bf16(qa[u][hh], dsb[u][hh], dk_acc[db]);
                    }
            }
        }
    };

    // one step = two visited query tiles, one per LDS stage
    auto step = [&](auto masked, int t) __attribute__((always_inline)) {
        if (t + 1 < n_vis)
            issue(qtile(t + 1), q1s, g1s, l1s, d1s);
        compute(masked, qtile(t), q0s, g0s, l0s, d0s);
        wait_vmem();
        __syncthreads();
        if (t + 1 < n_vis) {
            if (t + 2 < n_vis)
                issue(qtile(t + 2), q0s, g0s, l0s, d0s);
            compute(masked, qtile(t + 1), q1s, g1s, l1s, d1s);
            wait_vmem();
            __syncthreads();
        }
    };
    if (n_vis > 0)
        issue(qtile(0), q0s, g0s, l0s, d0s);
    wait_vmem();
    __syncthreads();
    if (n_vis > 0)
        step(std::integral_constant<bool, CAUSAL>{}, 0);   // the diagonal tiles (causal)
    for (int t = 2; t < n_vis; t += 2)
        step(std::false_type{}, t);

    // dK = scale * dS^T Q, dV = P^T dO; rows of padded keys are 0
    if (key >= kv_len) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            dk_acc[db] = f32x16{};
            dv_acc[db] = f32x16{};
        }
    }
    if (key < N) {
        bf16 *dK = (bf16 *)p.dk + head_off + (size_t)key * D;
        bf16 *dV = (bf16 *)p.dv + head_off + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 kv4, vv4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kv4[e] = (bf16)(dk_acc[db][4 * g + e] * p.scale);
                    vv4[e] = (bf16)dv_acc[db][4 * g + e];
                }
                if constexpr (DO_DK)
                    *(bf16x4 *)(dK + db * 32 + 8 * g + 4 * hf) = kv4;
                if constexpr (DO_DV)
                    *(bf16x4 *)(dV + db * 32 + 8 * g + 4 * hf) = vv4;
            }
    }
}

// dQ: queries outer ---------------------------------------------------------
// K and V tiles reach LDS by direct buffer->LDS loads into two stages.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, (D == 256 || (D == 128 && !CAUSAL)) ? 1 : 2) void bwd_dq_kernel(BwdArgs p, float c_log2)
{
    constexpr int BR = 128, BC = 64;
    constexpr int KSTEPS = D / 16;
    constexpr int NKC = BC / 32;
    constexpr int NDB = D / 32;

    __shared__ __attribute__((aligned(1024))) bf16 k0s[BC * D];
    __shared__ __attribute__((aligned(1024))) bf16 v0s[BC * D];
    __shared__ __attribute__((aligned(1024))) bf16 k1s[BC * D];
    __shared__ __attribute__((aligned(1024))) bf16 v1s[BC * D];

    const int N = p.N;
    const int n_qblk = (N + BR - 1) / BR;
    const int total = p.B * p.H * n_qblk;
    const int w = xcd_remap(blockIdx.x, total);
    const int bh = w / n_qblk;
    int qb = w % n_qblk;
    if (CAUSAL)
        qb = n_qblk - 1 - qb;
    const int b = bh / p.H;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int q0 = qb * BR;
    const int wq0 = q0 + wave * 32;
    const int qrow = wq0 + l32;

    const size_t head_off = (size_t)bh * N * D;
    const bf16 *Q = (const bf16 *)p.q + head_off;
    const bf16 *dO = (const bf16 *)p.dout + head_off;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc((const bf16 *)p.k + head_off, N, D);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc((const bf16 *)p.v + head_off, N, D);

    int kv_len = N;
    if (p.kv_lens) {
        kv_len = p.kv_lens[b];
        kv_len = kv_len < 0 ? 0 : (kv_len > N ? N : kv_len);
    }

    bf16x8 qreg[KSTEPS], greg[KSTEPS];
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
        if (qrow < N) {
            qreg[st] = *(const bf16x8 *)(Q + (size_t)qrow * D + st * 16 + hf * 8);
            greg[st] = *(const bf16x8 *)(dO + (size_t)qrow * D + st * 16 + hf * 8);
        } else {
            qreg[st] = bf16x8{};
            greg[st] = bf16x8{};
        }
    }
    float lse2 = INFINITY, dval = 0.f;
    if (qrow < N) {
        lse2 = p.lse2[(size_t)bh * N + qrow];
        dval = p.dvec[(size_t)bh * N + qrow];
    }

    f32x16 dq_acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        dq_acc[db] = f32x16{};

    // the key tiles visited: dense, 0 .. up to the diagonal / key length;
    // block-sparse, the two tiles of every nonzero block of this query
    // block's mask row
    __shared__ int blist[SPARSE ? MAX_MASK_BLOCKS : 1];
    __shared__ int bcount;
    int n_tiles;
    if constexpr (SPARSE) {
        if (wave == 0)
            list_nonzero(p.mask + (size_t)qb * p.nb, p.nb, 1, blist, &bcount);
        __syncthreads();
        n_tiles = __builtin_amdgcn_readfirstlane(bcount) * (128 / BC);
    } else {
        int kv_end = kv_len;
        if (CAUSAL)
            kv_end = min(kv_end, q0 + BR);
        n_tiles = (kv_end + BC - 1) / BC;
    }
    auto ktile = [&](int t) __attribute__((always_inline)) -> int {
        if constexpr (SPARSE)
            return __builtin_amdgcn_readfirstlane(blist[t / (128 / BC)]) * (128 / BC) + t % (128 / BC);
        else
            return t;
    };

    TileDma<BC, D, 4> dma;
    dma.init(wave);
    auto issue = [&](int t, bf16 *kd, bf16 *vd) __attribute__((always_inline)) {
        dma.issue(krs, ktile(t) * BC, kd, wave);
        dma.issue(vrs, ktile(t) * BC, vd, wave);
    };

    // MASKED instances handle the trailing tiles that cross the causal
    // diagonal or the key length; the main loop runs the unmasked instance
    auto compute = [&](auto masked, int t, const bf16 *kt, const bf16 *vt) __attribute__((always_inline)) {
        const int kbase = ktile(t) * BC;
        if (CAUSAL && kbase > wq0 + 31)
            return;
        const bool need_mask =
            decltype(masked)::value && ((kbase + BC > kv_len) || (CAUSAL && kbase + BC - 1 > wq0));
        // one 32-key chunk at a time: S^T, dP^T, dS^T, then dQ^T += K^T dS^T
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            // operands two k-steps ahead of the products; the group barriers
            // fix the order (reads for step st+2 right after the MFMAs of st)
            f32x16 s = f32x16{}, dp = f32x16{};
            constexpr int PF = 2;
            // priority up while this wave issues matrix products, so that the
            // other wave on the SIMD runs its vector work in the gaps
            __builtin_amdgcn_s_setprio(1);
            bf16x8 ka[KSTEPS], va[KSTEPS];
#pragma unroll
            for (int st = 0; st < PF; ++st) {
                ka[st] = ld_row8<D>(kt, kc * 32 + l32, st * 16 + hf * 8);
                va[st] = ld_row8<D>(vt, kc * 32 + l32, st * 16 + hf * 8);
            }
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                s = mfma_bf16(ka[st], qreg[st], s);
                dp = mfma_bf16(va[st], greg[st], dp);
                if (st + PF < KSTEPS) {
                    ka[st + PF] = ld_row8<D>(kt, kc * 32 + l32, (st + PF) * 16 + hf * 8);
                    va[st + PF] = ld_row8<D>(vt, kc * 32 + l32, (st + PF) * 16 + hf * 8);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);      // DS reads
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);       // MFMA
                if (st + PF < KSTEPS)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS reads
            }
            __builtin_amdgcn_s_setprio(0);
            bf16x8 dsb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kj = kbase + kc * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
                float pv = exp2_hw(fmaf(s[i], c_log2, -lse2));
                if (need_mask && (kj >= kv_len || (CAUSAL && kj > qrow)))
                    pv = 0.f;
                dsb[i / 8][i % 8] = (bf16)(pv * (dp[i] - dval));
            }
            bf16x8 kta[NDB][2];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    kta[db][hh] = ld_tr8<D>(kt, kc * 32 + hh * 16, db * 32);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    dq_acc[db] = mfma_bf16(kta[db][hh], dsb[hh], dq_acc[db]);
            __builtin_amdgcn_s_setprio(0);
        }
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
    // leading tiles that no wave needs to mask
    int n_plain = n_tiles;
    if constexpr (!SPARSE) {
        n_plain = min(n_tiles, kv_len / BC);
        if (CAUSAL)
            n_plain = min(n_plain, (q0 + 1) / BC);
    }
    const int t_mask = n_plain & ~1;
    if (n_tiles > 0)
        issue(0, k0s, v0s);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < t_mask; t += 2)
        step(std::false_type{}, t);
    for (int t = t_mask; t < n_tiles; t += 2)
        step(std::true_type{}, t);

    if (qrow < N) {
        bf16 *dQ = (bf16 *)p.dq + head_off + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v4[e] = (bf16)(dq_acc[db][4 * g + e] * p.scale);
                *(bf16x4 *)(dQ + db * 32 + 8 * g + 4 * hf) = v4;
            }
    }
}

template <int D>
hipError_t launch_dot(const BwdArgs &a, hipStream_t s)
{
    const int rows = a.B * a.H * a.N;
    constexpr int RPB = 256 / (D / 8);
    const bf16 *o = (const bf16 *)a.o, *g = (const bf16 *)a.dout;
    const float *lse = a.lse;
    float *dvec = a.dvec, *lse2 = a.lse2;
    void *kargs[] = {&o, &g, &lse, &dvec, &lse2, (void *)&rows};
    return hipLaunchKernel((const void *)&bwd_dot_kernel<D>, dim3((rows + RPB - 1) / RPB), dim3(256),
                           kargs, 0, s);
}

template <int D, bool CAUSAL, bool SPARSE, int MODE>
hipError_t launch_dkdv_mode(const BwdArgs &a, hipStream_t s)
{
    BwdArgs args = a;
    float c = a.scale * kLog2e;
    void *kargs[] = {&args, &c};
    const int n_kb = (a.N + 127) / 128;
    return hipLaunchKernel((const void *)&bwd_dkdv_kernel<D, CAUSAL, SPARSE, MODE>,
                           dim3(a.B * a.H * n_kb), dim3(256), kargs, 0, s);
}

// d = 64, 128: one launch for dK and dV; d = 256: a dV launch and a dK launch
template <int D, bool CAUSAL, bool SPARSE>
hipError_t launch_dkdv(const BwdArgs &a, hipStream_t s)
{
    if constexpr (D == 256) {
        hipError_t e = launch_dkdv_mode<D, CAUSAL, SPARSE, 1>(a, s);
        return e == hipSuccess ? launch_dkdv_mode<D, CAUSAL, SPARSE, 2>(a, s) : e;
    } else {
        return launch_dkdv_mode<D, CAUSAL, SPARSE, 0>(a, s);
    }
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t launch_dq(const BwdArgs &a, hipStream_t s)
{
    BwdArgs args = a;
    float c = a.scale * kLog2e;
    void *kargs[] = {&args, &c};
    const int n_qb = (a.N + 127) / 128;
    return hipLaunchKernel((const void *)&bwd_dq_kernel<D, CAUSAL, SPARSE>, dim3(a.B * a.H * n_qb),
                           dim3(256), kargs, 0, s);
}

template <int D>
hipError_t launch_d(const BwdArgs &a, bool causal, bool sparse, BwdStage stage, hipStream_t s)
{
    switch (stage) {
    case BwdStage::Dot:
        return launch_dot<D>(a, s);
    case BwdStage::DkDv:
        if (sparse)
            return launch_dkdv<D, false, true>(a, s);
        return causal ? launch_dkdv<D, true, false>(a, s) : launch_dkdv<D, false, false>(a, s);
    case BwdStage::Dq:
        if (sparse)
            return launch_dq<D, false, true>(a, s);
        return causal ? launch_dq<D, true, false>(a, s) : launch_dq<D, false, false>(a, s);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_bwd_stage(const BwdArgs &a, int d, bool causal, bool sparse, BwdStage stage,
                            hipStream_t s)
{
    if (d == 64)
        return launch_d<64>(a, causal, sparse, stage, s);
    if (d == 128)
        return launch_d<128>(a, causal, sparse, stage, s);
    if (d == 256)
        return launch_d<256>(a, causal, sparse, stage, s);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16(const BwdArgs &a, int d, bool causal, bool sparse, hipStream_t s)
{
    hipError_t e = launch_bwd_stage(a, d, causal, sparse, BwdStage::Dot, s);
    if (e == hipSuccess)
        e = launch_bwd_stage(a, d, causal, sparse, BwdStage::DkDv, s);
    if (e == hipSuccess)
        e = launch_bwd_stage(a, d, causal, sparse, BwdStage::Dq, s);
    return e;
}

} // namespace fa
