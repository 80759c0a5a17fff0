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
//   2. bwd_dkdv_kernel (fa_bwd_dkdv.hip, a translation unit of its own so it
//      can take its own scheduling flags): keys outer.  A workgroup owns 128
//      keys of one (b, h) (32 per wave, held in registers as MFMA operands)
//      and walks the query tiles, accumulating dK and dV in registers.
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
        return launch_bwd_dkdv(a, D, causal, sparse, s);
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
