// fa_bwd_dkdv.hip -- the dK, dV kernel of the backward pass (gfx950).
//
// The backward pass and the MFMA layouts of its kernels are described at the
// top of fa_bwd.hip; this kernel sits in a file of its own because it builds
// with a different instruction-scheduling strategy than the rest (chosen by
// measurement: the dQ kernel is faster with the default one).  It reads the
// workspace the preprocessing kernel of fa_bwd.hip fills: D_i = dO_i . O_i
// and LSE_i log2(e) per query row.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {

namespace {

// dK, dV: keys outer ------------------------------------------------------
// Q and dO tiles (and their rows' LSE and D) reach LDS by direct buffer->LDS
// loads into two stages; the loop is unrolled by two.  Query rows past N read
// as zeros (Q, dO, LSE, D all 0), which makes their dS and P^T dO terms 0.
//
// MODE 0 computes dK and dV together.  At d = 256 the K, V operands and the
// two accumulators of a wave's 32 keys do not fit one wave's registers, so
// the work is split over two launches: MODE 1 (dV only: S, P, dV^T += dO^T P)
// and MODE 2 (dK only: S, dP, dS, dK^T += Q^T dS), recomputing S once more.
template <int D, int BQ, bool CAUSAL, bool SPARSE, int MODE>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(BwdArgs p, float c_log2)
{
    constexpr bool DO_DV = MODE != 2, DO_DK = MODE != 1;
    constexpr int BKV = 128;
    static_assert(BQ == 64 || BQ == 128, "query tile");
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
    int bh, kb;
    if (CAUSAL) {
        // low key blocks have the most work; Q and dO tiles are streamed
        causal_item(blockIdx.x, p.B * p.H, n_kb, l2_group(N, 4 * D), bh, kb);
    } else {
        const int w = xcd_remap(blockIdx.x, total);
        bh = w / n_kb;
        kb = w % n_kb;
    }
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
        // 64 rows of LSE (even waves) and of D (odd waves) per instruction
        const int part = wave >> 1;
        if (part < BQ / 64) {
            if ((wave & 1) == 0)
                buffer_to_lds4(lrs, ld + part * 64, lane * 4, (qbase + part * 64) * 4);
            else if (DO_DK)
                buffer_to_lds4(drs, dd + part * 64, lane * 4, (qbase + part * 64) * 4);
        }
    };

    // MASKED applies the causal mask.  Only the query tiles that hold this
    // workgroup's diagonal (the first visited: qbase = k0 and, with 64-row
    // tiles, k0 + 64) need it; the first step is peeled off the main loop
    // below.  Key padding needs no
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

template <int D, int BQ, bool CAUSAL, bool SPARSE, int MODE>
hipError_t launch_dkdv_mode(const BwdArgs &a, hipStream_t s)
{
    BwdArgs args = a;
    float c = a.scale * kLog2e;
    void *kargs[] = {&args, &c};
    const int n_kb = (a.N + 127) / 128;
    return hipLaunchKernel((const void *)&bwd_dkdv_kernel<D, BQ, CAUSAL, SPARSE, MODE>,
                           dim3(a.B * a.H * n_kb), dim3(256), kargs, 0, s);
}

// d = 64, 128: one launch for dK and dV; d = 256: a dV launch and a dK launch.
// Query tiles of 64 rows, or 128 at d <= 128 (two stages of 128-row Q and
// dO tiles at d = 256 would need 256 KB of LDS).
template <int D, bool CAUSAL, bool SPARSE>
hipError_t launch_dkdv(const BwdArgs &a, hipStream_t s)
{
    if constexpr (D == 256) {
        if (a.tile_q != 0 && a.tile_q != 64)
            return hipErrorInvalidValue;
        hipError_t e = launch_dkdv_mode<D, 64, CAUSAL, SPARSE, 1>(a, s);
        return e == hipSuccess ? launch_dkdv_mode<D, 64, CAUSAL, SPARSE, 2>(a, s) : e;
    } else {
        if (a.tile_q == 128)
            return launch_dkdv_mode<D, 128, CAUSAL, SPARSE, 0>(a, s);
        if (a.tile_q != 0 && a.tile_q != 64)
            return hipErrorInvalidValue;
        return launch_dkdv_mode<D, 64, CAUSAL, SPARSE, 0>(a, s);
    }
}

} // namespace

hipError_t launch_bwd_dkdv(const BwdArgs &a, int d, bool causal, bool sparse, hipStream_t s)
{
    auto run = [&](auto dc) -> hipError_t {
        constexpr int D = decltype(dc)::value;
        if (sparse)
            return launch_dkdv<D, false, true>(a, s);
        return causal ? launch_dkdv<D, true, false>(a, s) : launch_dkdv<D, false, false>(a, s);
    };
    if (d == 64)
        return run(std::integral_constant<int, 64>{});
    if (d == 128)
        return run(std::integral_constant<int, 128>{});
    if (d == 256)
        return run(std::integral_constant<int, 256>{});
    return hipErrorInvalidValue;
}

} // namespace fa
