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
//   1. bwd_dot_kernel: D_i = dO_i . O_i (fp32) into the workspace.
//   2. bwd_dkdv_kernel: keys outer.  A workgroup owns 128 keys of one
//      (b, h) (32 per wave, held in registers as MFMA operands) and walks the
//      query tiles, accumulating dK and dV in registers.
//   3. bwd_dq_kernel: queries outer.  A workgroup owns 128 queries and walks
//      the key tiles, accumulating dQ in registers.
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

#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {

namespace {

// D_i = dO_i . O_i in fp32 -----------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const bf16 *__restrict__ o,
                                                      const bf16 *__restrict__ dout,
                                                      float *__restrict__ dvec, int rows)
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
    if (r < rows && threadIdx.x % CPR == 0)
        dvec[r] = acc;
}

// dK, dV: keys outer ------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs p, float c_log2)
{
    constexpr int BKV = 128, BQ = 64;
    constexpr int KSTEPS = D / 16;
    constexpr int NQC = BQ / 32;           // 32-query chunks per tile
    constexpr int NDB = D / 32;

    __shared__ __attribute__((aligned(16))) bf16 qs[2][BQ * D];
    __shared__ __attribute__((aligned(16))) bf16 dos[2][BQ * D];
    __shared__ __attribute__((aligned(16))) float lse_s[2][BQ];
    __shared__ __attribute__((aligned(16))) float dd_s[2][BQ];

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
    const bf16 *Q = (const bf16 *)p.q + head_off;
    const bf16 *K = (const bf16 *)p.k + head_off;
    const bf16 *V = (const bf16 *)p.v + head_off;
    const bf16 *dO = (const bf16 *)p.dout + head_off;
    const float *LSE = p.lse + (size_t)bh * N;
    const float *Dv = p.dvec + (size_t)bh * N;

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
            vreg[st] = *(const bf16x8 *)(V + (size_t)key * D + st * 16 + hf * 8);
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

    const int n_qt = (N + BQ - 1) / BQ;
    const int qt_begin = (CAUSAL ? k0 / BQ : 0);
    const int qt_end = (k0 < kv_len) ? n_qt : qt_begin;   // no allowed key: nothing to do
    const bool wave_live = wk0 < kv_len;

    TileStage<BQ, D> qst, gst;
    float lse_r = INFINITY, dd_r = 0.f;    // threads < BQ stage one row's LSE and D
    const __amdgpu_buffer_rsrc_t qrs = head_rsrc(Q, N, D), grs = head_rsrc(dO, N, D);
    auto load_tile = [&](int it) {
        const int qbase = it * BQ;
        qst.load(qrs, qbase);
        gst.load(grs, qbase);
        if (tid < BQ) {
            const int qi = qbase + tid;
            lse_r = INFINITY;              // rows past N: P = 0
            dd_r = 0.f;
            if (qi < N) {
                const float l = LSE[qi];
                lse_r = (l == -INFINITY) ? INFINITY : l * kLog2e;
                dd_r = Dv[qi];
            }
        }
    };
    auto store_tile = [&](int buf) {
        qst.store(qs[buf]);
        gst.store(dos[buf]);
        if (tid < BQ) {
            lse_s[buf][tid] = lse_r;
            dd_s[buf][tid] = dd_r;
        }
    };

    if (qt_begin < qt_end) {
        load_tile(qt_begin);
        store_tile(0);
    }
    __syncthreads();

    for (int it = qt_begin; it < qt_end; ++it) {
        const int buf = (it - qt_begin) & 1;
        const int qbase = it * BQ;
        if (it + 1 < qt_end)
            load_tile(it + 1);

        const bool skip = !wave_live || (CAUSAL && qbase + BQ - 1 < wk0);
        if (!skip) {
            f32x16 s[NQC], dp[NQC];
#pragma unroll
            for (int qc = 0; qc < NQC; ++qc) {
                s[qc] = f32x16{};
                dp[qc] = f32x16{};
#pragma unroll
                for (int st = 0; st < KSTEPS; ++st) {
                    s[qc] = mfma_bf16(ld_row8<D>(qs[buf], qc * 32 + l32, st * 16 + hf * 8), kreg[st], s[qc]);
                    dp[qc] = mfma_bf16(ld_row8<D>(dos[buf], qc * 32 + l32, st * 16 + hf * 8), vreg[st], dp[qc]);
                }
            }
            const bool need_mask = (CAUSAL && qbase < wk0 + 31) || (wk0 + 32 > kv_len);
            bf16x8 pb[NQC][2], dsb[NQC][2];
#pragma unroll
            for (int qc = 0; qc < NQC; ++qc)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int trow = qc * 32 + 8 * g + 4 * hf;
                    const f32x4 l4 = *(const f32x4 *)&lse_s[buf][trow];
                    const f32x4 d4 = *(const f32x4 *)&dd_s[buf][trow];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * g + e;
                        float pv = exp2_hw(fmaf(s[qc][i], c_log2, -l4[e]));
                        if (need_mask && (key >= kv_len || (CAUSAL && key > qbase + trow + e)))
                            pv = 0.f;
                        const float ds = pv * (dp[qc][i] - d4[e]);
                        pb[qc][i / 8][i % 8] = (bf16)pv;
                        dsb[qc][i / 8][i % 8] = (bf16)ds;
                    }
                }
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int qc = 0; qc < NQC; ++qc)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        dv_acc[db] = mfma_bf16(ld_tr8<D>(dos[buf], qc * 32 + hh * 16, db * 32), pb[qc][hh], dv_acc[db]);
                        dk_acc[db] = mfma_bf16(ld_tr8<D>(qs[buf], qc * 32 + hh * 16, db * 32), dsb[qc][hh], dk_acc[db]);
                    }
        }
        if (it + 1 < qt_end)
            store_tile(buf ^ 1);
        __syncthreads();
    }

    // dK = scale * dS^T Q, dV = P^T dO; rows of padded keys stay 0
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
                *(bf16x4 *)(dK + db * 32 + 8 * g + 4 * hf) = kv4;
                *(bf16x4 *)(dV + db * 32 + 8 * g + 4 * hf) = vv4;
            }
    }
}

// dQ: queries outer ---------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs p, float c_log2)
{
    constexpr int BR = 128, BC = 64;
    constexpr int KSTEPS = D / 16;
    constexpr int NKC = BC / 32;
    constexpr int NDB = D / 32;

    __shared__ __attribute__((aligned(16))) bf16 ks[2][BC * D];
    __shared__ __attribute__((aligned(16))) bf16 vs[2][BC * D];

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
    const bf16 *K = (const bf16 *)p.k + head_off;
    const bf16 *V = (const bf16 *)p.v + head_off;
    const bf16 *dO = (const bf16 *)p.dout + head_off;

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
        const float l = p.lse[(size_t)bh * N + qrow];
        lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
        dval = p.dvec[(size_t)bh * N + qrow];
    }

    f32x16 dq_acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        dq_acc[db] = f32x16{};

    int kv_end = kv_len;
    if (CAUSAL)
        kv_end = min(kv_end, q0 + BR);
    const int n_tiles = (kv_end + BC - 1) / BC;

    TileStage<BC, D> kst, vst;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc(K, N, D), vrs = head_rsrc(V, N, D);
    auto load_tile = [&](int t) {
        kst.load(krs, t * BC);
        vst.load(vrs, t * BC);
    };
    if (n_tiles > 0) {
        load_tile(0);
        kst.store(ks[0]);
        vst.store(vs[0]);
    }
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        const int kbase = t * BC;
        if (t + 1 < n_tiles)
            load_tile(t + 1);

        const bool skip = CAUSAL && kbase > wq0 + 31;
        if (!skip) {
            f32x16 s[NKC], dp[NKC];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                s[kc] = f32x16{};
                dp[kc] = f32x16{};
#pragma unroll
                for (int st = 0; st < KSTEPS; ++st) {
                    s[kc] = mfma_bf16(ld_row8<D>(ks[buf], kc * 32 + l32, st * 16 + hf * 8), qreg[st], s[kc]);
                    dp[kc] = mfma_bf16(ld_row8<D>(vs[buf], kc * 32 + l32, st * 16 + hf * 8), greg[st], dp[kc]);
                }
            }
            const bool need_mask = (kbase + BC > kv_len) || (CAUSAL && kbase + BC - 1 > wq0);
            bf16x8 dsb[NKC][2];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kj = kbase + kc * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
                    float pv = exp2_hw(fmaf(s[kc][i], c_log2, -lse2));
                    if (need_mask && (kj >= kv_len || (CAUSAL && kj > qrow)))
                        pv = 0.f;
                    dsb[kc][i / 8][i % 8] = (bf16)(pv * (dp[kc][i] - dval));
                }
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        dq_acc[db] = mfma_bf16(ld_tr8<D>(ks[buf], kc * 32 + hh * 16, db * 32), dsb[kc][hh], dq_acc[db]);
        }
        if (t + 1 < n_tiles) {
            kst.store(ks[buf ^ 1]);
            vst.store(vs[buf ^ 1]);
        }
        __syncthreads();
    }

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
    float *dvec = a.dvec;
    void *kargs[] = {&o, &g, &dvec, (void *)&rows};
    return hipLaunchKernel((const void *)&bwd_dot_kernel<D>, dim3((rows + RPB - 1) / RPB), dim3(256),
                           kargs, 0, s);
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv(const BwdArgs &a, hipStream_t s)
{
    BwdArgs args = a;
    float c = a.scale * kLog2e;
    void *kargs[] = {&args, &c};
    const int n_kb = (a.N + 127) / 128;
    return hipLaunchKernel((const void *)&bwd_dkdv_kernel<D, CAUSAL>, dim3(a.B * a.H * n_kb),
                           dim3(256), kargs, 0, s);
}

template <int D, bool CAUSAL>
hipError_t launch_dq(const BwdArgs &a, hipStream_t s)
{
    BwdArgs args = a;
    float c = a.scale * kLog2e;
    void *kargs[] = {&args, &c};
    const int n_qb = (a.N + 127) / 128;
    return hipLaunchKernel((const void *)&bwd_dq_kernel<D, CAUSAL>, dim3(a.B * a.H * n_qb),
                           dim3(256), kargs, 0, s);
}

} // namespace

hipError_t launch_bwd_stage(const BwdArgs &a, int d, bool causal, BwdStage stage, hipStream_t s)
{
    if (d != 64 && d != 128)
        return hipErrorInvalidValue;
    switch (stage) {
    case BwdStage::Dot:
        return d == 64 ? launch_dot<64>(a, s) : launch_dot<128>(a, s);
    case BwdStage::DkDv:
        if (d == 64)
            return causal ? launch_dkdv<64, true>(a, s) : launch_dkdv<64, false>(a, s);
        return causal ? launch_dkdv<128, true>(a, s) : launch_dkdv<128, false>(a, s);
    case BwdStage::Dq:
        if (d == 64)
            return causal ? launch_dq<64, true>(a, s) : launch_dq<64, false>(a, s);
        return causal ? launch_dq<128, true>(a, s) : launch_dq<128, false>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16(const BwdArgs &a, int d, bool causal, hipStream_t s)
{
    hipError_t e = launch_bwd_stage(a, d, causal, BwdStage::Dot, s);
    if (e == hipSuccess)
        e = launch_bwd_stage(a, d, causal, BwdStage::DkDv, s);
    if (e == hipSuccess)
        e = launch_bwd_stage(a, d, causal, BwdStage::Dq, s);
    return e;
}

} // namespace fa
