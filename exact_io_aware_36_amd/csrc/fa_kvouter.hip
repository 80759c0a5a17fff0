// fa_kvouter.hip -- the key/value-outer loop order, kept as an IO ablation.
//
// "FlashAttention: Mathematical Foundations, IO-Aware Tiling, Online Softmax,
// and Recomputation Dynamics", section "IO-Aware Tiling Algorithm" (its
// Algorithm 1), and "01 · FlashAttention" (attention-lab), step 5: the
// outer loop walks key/value blocks and the inner loop query blocks, so each
// query block's output accumulator and running statistics (O_i, l_i, m_i)
// are read from and written back to HBM once per key/value block.  That is
// what the pages' HBM accounting counts (4Nd + 2N^2 d^2 / M elements per
// head, against 2N^2 + 4Nd for standard attention).  The production forward
// (fa_fwd.hip) keeps O, l and m in registers for the whole key loop instead;
// this file exists to measure what that buys on MI355X.
//
// MI355X form: the key/value loop is a sequence of launches, one per 64-key
// block j, each a grid over (b, h, 128-row query block).  A workgroup loads
// K_j and V_j into LDS, its queries' Q into registers and their fp32 O, l, m
// from the workspace, applies the two-block update of the article's section
// "Incremental Online Updates" (exact maximum, no lazy threshold), and
// writes them back.  A last launch divides O by l, converts to bf16 and
// writes LSE.  Same MFMA layout as the forward (S^T = K Q^T, lane = query).
#include <hip/hip_runtime.h>
#include <math.h>

#include "fa_internal.h"
#include "fa_kvouter.h"
#include "fa_tile.h"

namespace fa {

namespace {

constexpr int KV_BR = 128, KV_BC = 64;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void kvouter_step_kernel(KvOuterArgs p, int j, float c_log2)
{
    constexpr int KSTEPS = D / 16, NKC = KV_BC / 32, NDB = D / 32;
    __shared__ __attribute__((aligned(1024))) bf16 ks[KV_BC * D];
    __shared__ __attribute__((aligned(1024))) bf16 vs[KV_BC * D];

    const int N = p.N;
    const int n_qblk = (N + KV_BR - 1) / KV_BR;
    const int bh = blockIdx.x / n_qblk, qb = blockIdx.x % n_qblk;
    const int q0 = qb * KV_BR, kbase = j * KV_BC;
    if (CAUSAL && kbase > q0 + KV_BR - 1)
        return;                               // every key of the block is masked: nothing changes
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int wq0 = q0 + wave * 32, qrow = wq0 + l32;

    const size_t head_off = (size_t)bh * N * D;
    {
        TileStage<KV_BC, D> kst, vst;
        kst.load(head_rsrc((const bf16 *)p.k + head_off, N, D), kbase);
        vst.load(head_rsrc((const bf16 *)p.v + head_off, N, D), kbase);
        kst.store(ks);
        vst.store(vs);
    }
    __syncthreads();
    if (CAUSAL && kbase > wq0 + 31)
        return;                               // this wave's rows see none of these keys

    bf16x8 qreg[KSTEPS];
    const bf16 *Q = (const bf16 *)p.q + head_off;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
        qreg[s] = qrow < N ? *(const bf16x8 *)(Q + (size_t)qrow * D + s * 16 + hf * 8) : bf16x8{};

    // running state of this lane's query from the workspace (block 0 starts it)
    const size_t srow = (size_t)bh * N + (qrow < N ? qrow : 0);
    float *ow = p.o_acc + srow * D;
    f32x16 oacc[NDB];
    float m = -INFINITY, l = 0.f;
    if (j > 0) {
        m = p.m[srow];
        l = p.l[srow];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 v4 = *(const f32x4 *)(ow + db * 32 + 8 * g + 4 * hf);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    oacc[db][4 * g + e] = v4[e];
            }
    } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            oacc[db] = f32x16{};
    }

    // S^T = K_j Q^T
    f32x16 s[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        s[kc] = f32x16{};
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
            s[kc] = mfma_bf16(ld_row8<D>(ks, kc * 32 + l32, st * 16 + hf * 8), qreg[st], s[kc]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = kbase + kc * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
            if (key >= N || (CAUSAL && key > qrow))
                s[kc][i] = -INFINITY;
            mx = fmaxf(mx, s[kc][i]);
        }
    // two-block update: m' = max(m, tile max), rescale l and O by 2^(m - m')
    const float m_new = fmaxf(m, pair_max(mx) * c_log2);
    const float alpha = exp2_hw(m - m_new);           // 0 when m = -inf
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float rs = 0.f;
    bf16x8 pb[NKC][2];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float pv = exp2_hw(fmaf(s[kc][i], c_log2, -m_use));
            rs += pv;
            pb[kc][i / 8][i % 8] = (bf16)pv;
        }
    l = l * alpha + pair_sum(rs);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        oacc[db] *= alpha;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                oacc[db] = mfma_bf16(ld_tr8<D>(vs, kc * 32 + hh * 16, db * 32), pb[kc][hh], oacc[db]);
    }

    // back to HBM
    if (qrow < N) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v4[e] = oacc[db][4 * g + e];
                *(f32x4 *)(ow + db * 32 + 8 * g + 4 * hf) = v4;
            }
        if (hf == 0) {
            p.m[srow] = m_new;
            p.l[srow] = l;
        }
    }
}

// O = O_acc / l in bf16, LSE = ln 2 (m + log2 l); one thread per 8 elements
template <int D>
__global__ __launch_bounds__(256) void kvouter_final_kernel(KvOuterArgs p)
{
    constexpr int TPR = D / 8;                 // threads per row
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)p.B * p.H * p.N;
    const int64_t row = t / TPR;
    if (row >= rows)
        return;
    const int c = (int)(t % TPR) * 8;
    const float l = p.l[row], m = p.m[row];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16x8 ov;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        ov[e] = (bf16)(p.o_acc[row * D + c + e] * inv);
    *(bf16x8 *)((bf16 *)p.o + row * D + c) = ov;
    if (c == 0)
        p.lse[row] = l > 0.f ? kLn2 * (m + __log2f(l)) : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch_kvouter_d(const KvOuterArgs &a, hipStream_t s)
{
    const int n_qblk = (a.N + KV_BR - 1) / KV_BR;
    const int n_kblk = (a.N + KV_BC - 1) / KV_BC;
    const dim3 grid((unsigned)(a.B * a.H * n_qblk)), block(256);
    KvOuterArgs args = a;
    float c = a.scale * kLog2e;
    for (int j = 0; j < n_kblk; ++j) {
        void *kargs[] = {&args, &j, &c};
        const hipError_t e = hipLaunchKernel((const void *)&kvouter_step_kernel<D, CAUSAL>, grid, block,
                                             kargs, 0, s);
        if (e != hipSuccess)
            return e;
    }
    const int64_t threads = (int64_t)a.B * a.H * a.N * (D / 8);
    void *fargs[] = {&args};
    return hipLaunchKernel((const void *)&kvouter_final_kernel<D>, dim3((unsigned)((threads + 255) / 256)),
                           block, fargs, 0, s);
}

} // namespace

hipError_t launch_fwd_kvouter(const KvOuterArgs &a, int d, bool causal, hipStream_t s)
{
    if (d == 64)
        return causal ? launch_kvouter_d<64, true>(a, s) : launch_kvouter_d<64, false>(a, s);
    if (d == 128)
        return causal ? launch_kvouter_d<128, true>(a, s) : launch_kvouter_d<128, false>(a, s);
    return hipErrorInvalidValue;
}

} // namespace fa
