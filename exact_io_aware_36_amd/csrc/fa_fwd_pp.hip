// fa_fwd_pp.hip -- the bf16 forward attention kernel in two alternating wave
// groups (gfx950).
//
// Same computation as fwd_bf16_kernel (fa_fwd.hip): exact attention
// O = softmax(scale Q K^T) V tile by tile with the running-statistics
// recurrence ("The Attention Matrix You Never Write Down", section "The
// running-statistics trick"; "FlashAttention: Mathematical Foundations,
// IO-Aware Tiling, Online Softmax, and Recomputation Dynamics", sections
// "Incremental Online Updates" and "IO-Aware Tiling Algorithm"), queries outer
// (the same article's "FlashAttention-2" section), storing only O and the
// per-row log-sum-exp.  The MFMA layouts are those of fwd_bf16_kernel: S^T =
// K Q^T puts one query per lane, P^T feeds O^T += V^T P^T from registers.
//
// What differs is how the work of a SIMD is laid out in time.  A workgroup of
// eight wave64s owns 256 query rows (32 per wave); waves w and w + 4 share a
// SIMD.  Waves 0-3 (group 0) and 4-7 (group 1) run the same loop one phase
// apart, every phase ending at a workgroup barrier, so that on each SIMD one
// wave runs matrix products while the other runs everything else:
//
//   MFMA block t:  S_t = K_t Q^T and O^T += V_{t-1}^T P_{t-1}^T from operands
//                  already in registers, with the LDS reads of the next MFMA
//                  block's operands (K_{t+1}, V_t) issued between the products.
//   VALU block t:  softmax of S_t -> P_t (masks, lazy rescale, row sums), the
//                  buffer->LDS copy of a tile NST - 1 ahead, a wait for the
//                  copy three tiles ahead.
//
// The exponentials and copies of one wave thus overlap the other wave's
// matrix products instead of taking turns with its own, and a block's reads
// have a whole phase to land before their products.  Key tiles of
// BC keys pass through NST LDS stages; a tile's stage is refilled once both
// groups have read its V (two phases after its K).  One workgroup per CU
// (512 threads, up to 256 registers per lane).
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {

namespace {

constexpr float TAU = 8.f;             // lazy-rescale threshold (log2 units)
constexpr float kPassLimit = 256.f;    // 2^TAU

// barrier after this wave's LDS reads have landed; its buffer->LDS copies stay
// in flight.  The scheduling fences keep ALU work on its side of the barrier.
__device__ __forceinline__ void phase_barrier_lds()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), seen by the compiler's own wait tracking
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void phase_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// One 16-byte-per-lane buffer->LDS copy (buffer_load_dwordx4 ... lds) to LDS
// byte address lds_addr, written as inline asm so that the compiler does not
// track it: it would otherwise make LDS reads of other stages wait for it.
// The kernel waits for its copies itself (vmcnt, then a barrier).  The
// instruction has no register results; M0 holds the LDS address and needs one
// wait state before the copy reads it.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, unsigned lds_addr, unsigned voff,
                                      int soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
                 : "memory", "m0");
}

// wait until at most N vector-memory loads of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_le()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

template <int D, int BC, int NST, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_pp_kernel(FwdArgs p, float c_log2)
{
    constexpr int BR = 256;                // query rows per workgroup
    constexpr int KSTEPS = D / 16;         // k-steps of S^T over d
    constexpr int NKC = BC / 32;           // 32-key chunks per tile
    constexpr int NDB = D / 32;            // 32-wide d blocks of O^T
    constexpr int TILE = BC * D;           // elements of one K or V tile
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int SEGS = TILE * 2 / 1024;  // 1 KB copy segments per K or V tile
    constexpr int PW = 2 * SEGS / 8;       // segments each wave copies per tile
    static_assert(PW * 8 == 2 * SEGS, "a tile's K and V must split evenly over eight waves");
    static_assert(NST >= 4, "three tiles are read while a fourth is copied");

    // stage s: K tile, then V tile.  One array per stage, addressed with
    // compile-time stage numbers, so the compiler can tell an LDS read of one
    // stage from the copies in flight into the others (a single array would
    // make it wait for every copy before each read).
    static_assert(NST <= 8 && NST % 2 == 0, "stages: an even number (V buffers alternate with the tile's parity)");
    __shared__ __attribute__((aligned(1024))) bf16 st0[2 * TILE];
    __shared__ __attribute__((aligned(1024))) bf16 st1[2 * TILE];
    __shared__ __attribute__((aligned(1024))) bf16 st2[2 * TILE];
    __shared__ __attribute__((aligned(1024))) bf16 st3[NST > 3 ? 2 * TILE : 1];
    __shared__ __attribute__((aligned(1024))) bf16 st4[NST > 4 ? 2 * TILE : 1];
    __shared__ __attribute__((aligned(1024))) bf16 st5[NST > 5 ? 2 * TILE : 1];
    __shared__ __attribute__((aligned(1024))) bf16 st6[NST > 6 ? 2 * TILE : 1];
    __shared__ __attribute__((aligned(1024))) bf16 st7[NST > 7 ? 2 * TILE : 1];
    auto stage = [&](auto sc) __attribute__((always_inline)) -> bf16 * {
        constexpr int S = decltype(sc)::value % NST;
        if constexpr (S == 0) return st0;
        else if constexpr (S == 1) return st1;
        else if constexpr (S == 2) return st2;
        else if constexpr (S == 3) return st3;
        else if constexpr (S == 4) return st4;
        else if constexpr (S == 5) return st5;
        else if constexpr (S == 6) return st6;
        else return st7;
    };

    // kept in a register: otherwise it is re-read from the argument buffer
    // inside the loop (and that read waits for the LDS reads in flight)
    asm volatile("" : "+s"(c_log2));
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
    const int grp = wave >> 2;               // waves w and w + 4 share a SIMD
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
    // tiles the workgroup walks, and the ones this wave computes
    const int kv_end = CAUSAL ? min(kv_len, q0 + BR) : kv_len;
    const int T = (kv_end + BC - 1) / BC;
    int T_w = wq0 < N ? T : 0;
    if (CAUSAL)
        T_w = min(T_w, (wq0 + 31) / BC + 1);     // tiles starting at or before its last query
    // leading tiles this wave needs no mask on
    int n_plain = min(T_w, kv_len / BC);
    if (CAUSAL)
        n_plain = min(n_plain, (wq0 + 1) / BC);

    bf16x8 qreg[KSTEPS];

    // ---- copies: segment wave + 8 i of a stage (K segments, then V's)
    unsigned dvoff[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int sl = (wave + 8 * i) % SEGS;
        const int chunk = sl * 64 + lane;
        const int row = chunk / CPR, pc = chunk % CPR;
        dvoff[i] = (unsigned)((row * D + ((pc ^ swz<D>(row)) << 3)) * 2);
    }
    auto issue_tile = [&](int j, bf16 *dst) __attribute__((always_inline)) {
        typedef bf16 __attribute__((address_space(3))) lds_bf16;
        const int soff = (int)((unsigned)(j * BC) * (unsigned)D * 2u);
        const unsigned base = (unsigned)(uintptr_t)(lds_bf16 *)dst;
#pragma unroll
        for (int i = 0; i < PW; ++i) {
            const int seg = wave + 8 * i;
            dma16(seg < SEGS ? krs : vrs, base + (unsigned)seg * 1024u, dvoff[i], soff);
        }
    };

    float m = -INFINITY;   // reference max (log2 units), same in both lane halves
    float lsum = 0.f;      // running sum, partial over this lane half's keys
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        oacc[db] = f32x16{};
    bf16x8 ka[NKC][KSTEPS];     // K_t operands (A of S^T)
    bf16x8 va[2][NDB][NKC][2];  // V^T operands (A of O^T += V^T P^T), tile t in va[t & 1]
    bf16x8 pb[NKC][2];          // P_t^T (B of the same)
    f32x16 s[NKC];              // S_t^T
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        pb[kc][0] = pb[kc][1] = bf16x8{};
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            va[0][db][kc][0] = va[0][db][kc][1] = va[1][db][kc][0] = va[1][db][kc][1] = bf16x8{};
    }

    // Per-lane byte offsets of the operand reads within a stage (the same in
    // every stage; the stage's own address goes into the instruction's
    // immediate offset).  K rows (ld_row8): k-step k of the 32 keys of chunk
    // kc at koff[k] + kc 32 D 2.  V^T (ld_tr8): d block db, rows row0 + {0..3}
    // and row0 + {8..11} of the lane's quarter at vof[db][0 / 1] + row0 D 2.
    unsigned koff[KSTEPS], vof[NDB][2];
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k)
        koff[k] = (unsigned)toff<D>(l32, k * 16 + hf * 8) * 2u;
    {
        const int r = 4 * (lane >> 5) + ((lane & 15) >> 2);
        const int c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            vof[db][0] = (unsigned)toff<D>(r, db * 32 + c) * 2u + (unsigned)(TILE * 2);
            vof[db][1] = (unsigned)toff<D>(r + 8, db * 32 + c) * 2u + (unsigned)(TILE * 2);
        }
    }
    // hide the offsets' values from the compiler at each step, so that it
    // adds the stage address per read instead of holding one sum per stage
    auto refresh_offsets = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k)
            asm volatile("" : "+v"(koff[k]));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            asm volatile("" : "+v"(vof[db][0]));
            asm volatile("" : "+v"(vof[db][1]));
        }
    };
    auto read_k = [&](const bf16 *stg) __attribute__((always_inline)) {
        const char *base = (const char *)stg;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k)
                ka[kc][k] = *(const bf16x8 *)(base + koff[k] + kc * 32 * D * 2);
    };
    // the n operand reads i0 .. i0 + n - 1 of K (in kc-major, k-step order)
    auto read_k_part = [&](const bf16 *stg, int i0, int n) __attribute__((always_inline)) {
        const char *base = (const char *)stg;
#pragma unroll
        for (int i = i0; i < i0 + n; ++i)
            ka[i / KSTEPS][i % KSTEPS] = *(const bf16x8 *)(base + koff[i % KSTEPS] + (i / KSTEPS) * 32 * D * 2);
    };
    // V^T operands of d block db into buffer vb
    auto read_v_block = [&](const bf16 *stg, int vb, int db) __attribute__((always_inline)) {
        typedef bf16x4 __attribute__((address_space(3))) lds_bf16x4;
        const char *base = (const char *)stg;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ro = (kc * 32 + hh * 16) * D * 2;
                const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + vof[db][0] + ro));
                const bf16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + vof[db][1] + ro));
                va[vb][db][kc][hh] = __builtin_shufflevector(a, b2, 0, 1, 2, 3, 4, 5, 6, 7);
            }
    };

    // Probabilities of S_t against the current reference m (see fa_fwd.hip:
    // the tile maximum is only needed when a partial row sum passes 2^TAU).
    auto softmax = [&](int t) __attribute__((always_inline)) {
        if (t >= n_plain) {
            const int kbase = t * BC;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kbase + kc * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
                    if (key >= kv_len || (CAUSAL && key > qrow))
                        s[kc][i] = -INFINITY;
                }
        }
        // row sums in four independent partial sums (a single chain of
        // dependent adds would stall the wave at every one of them)
        float rs = 0.f;
        bool slow = __any(m == -INFINITY);
        if (!slow) {
            // four partial sums, each started at its first probability (an add
            // to 0.0f is an instruction: the compiler keeps it for -0, which an
            // exponential never is)
            float r4[4];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = exp2_hw(fmaf(s[kc][i], c_log2, -m));
                    if (kc == 0 && i < 4)
                        r4[i] = pv;
                    else
                        r4[i % 4] += pv;
                    pb[kc][i / 8][i % 8] = (bf16)pv;
                }
            rs = (r4[0] + r4[1]) + (r4[2] + r4[3]);
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
            // four partial sums, each started at its first probability (an add
            // to 0.0f is an instruction: the compiler keeps it for -0, which an
            // exponential never is)
            float r4[4];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = exp2_hw(fmaf(s[kc][i], c_log2, -m_use));
                    if (kc == 0 && i < 4)
                        r4[i] = pv;
                    else
                        r4[i % 4] += pv;
                    pb[kc][i / 8][i % 8] = (bf16)pv;
                }
            rs = (r4[0] + r4[1]) + (r4[2] + r4[3]);
        }
        lsum += rs;
    };

    // MFMA block t: the products of S_t and of O^T += V_{t-1}^T P_{t-1}^T,
    // taken alternately (each product of the dependent S chain follows an
    // independent one), with the LDS reads of the next block's operands
    // spread over them: after the i-th S product has consumed ka[i], K_{t+1}'s
    // i-th operand goes into it, and V_t goes into the other V buffer.  VB is
    // the buffer of V_t (t & 1; the step's stage number has t's parity).  One
    // branch for the whole block: for t = 0 the P and V operands are still
    // zero (adding nothing), at t = T_w the S products and reads are wasted
    // once per wave, and waves past their last tile skip it.
    auto mfma_block = [&](int t, auto vbc, const bf16 *knext, const bf16 *vcur, bool reads)
                          __attribute__((always_inline)) {
        constexpr int VB = decltype(vbc)::value, PB = VB ^ 1;
        constexpr int NS = NKC * KSTEPS;          // S products
        constexpr int NP = NDB * NKC * 2;         // P V products
        static_assert(NS == NP, "one S product per P V product (D = 32 NKC KSTEPS / 2 ... )");
        typedef bf16x4 __attribute__((address_space(3))) lds_bf16x4;
        if (t <= T_w) {
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                s[kc] = f32x16{};
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int kc = i / KSTEPS, k = i % KSTEPS;            // S product i
                const int db = i / (NKC * 2), pc = (i / 2) % NKC, hh = i % 2;   // P V product i
                s[kc] = mfma_bf16(ka[kc][k], qreg[k], s[kc]);
                oacc[db] = mfma_bf16(va[PB][db][pc][hh], pb[pc][hh], oacc[db]);
                if (reads) {
                    ka[kc][k] = *(const bf16x8 *)((const char *)knext + koff[k] + kc * 32 * D * 2);
                    // V_t operand i: d block db, key chunk pc, half hh
                    const int ro = (pc * 32 + hh * 16) * D * 2;
                    const char *vb = (const char *)vcur;
                    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vb + vof[db][0] + ro));
                    const bf16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vb + vof[db][1] + ro));
                    va[VB][db][pc][hh] = __builtin_shufflevector(a, b2, 0, 1, 2, 3, 4, 5, 6, 7);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // One tile step in stage S (compile-time): MFMA block t (reading K_{t+1}
    // from stage S + 1 and V_t from stage S), then VALU block t: the copy of
    // tile t + NST - 1 into stage S + NST - 1 (that of tile t - 1, which both
    // groups have finished reading), the softmax of S_t, and a wait for tile
    // t + 3 before the closing barrier (the MFMA blocks of the next phases
    // read it).
    auto step = [&](int t, auto sc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        using S1 = std::integral_constant<int, S + 1>;
        using SF = std::integral_constant<int, S + NST - 1>;
        refresh_offsets();
        mfma_block(t, std::integral_constant<int, S & 1>{}, stage(S1{}), stage(sc), true);
        // the operand reads may still be in flight: their stages are not
        // refilled before two more phases, and their first use (the next
        // MFMA block) waits for them
        phase_barrier();
        issue_tile(min(t + NST - 1, T - 1), stage(SF{}));
        if (t < T_w)
            softmax(t);
        wait_vmem_le<(NST - 4) * PW>();
        phase_barrier();
    };

    if (T > 0) {
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using I4 = std::integral_constant<int, 4>;
        using I5 = std::integral_constant<int, 5>;
        using I6 = std::integral_constant<int, 6>;
        using I7 = std::integral_constant<int, 7>;
        // tiles 0, 1 and 2, then Q (the B operand of S^T = K Q^T), then a
        // wait the compiler can see for Q: it covers those tiles as well, and
        // leaves the compiler no load of its own outstanding in the loop
        issue_tile(0, stage(I0{}));
        issue_tile(min(1, T - 1), stage(I1{}));
        issue_tile(min(2, T - 1), stage(I2{}));
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) {
            if (qrow < N)
                qreg[k] = *(const bf16x8 *)(Q + (size_t)qrow * D + k * 16 + hf * 8);
            else
                qreg[k] = bf16x8{};
        }
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k)
            asm volatile("" : "+v"(qreg[k]));
        // tiles 3 .. NST-2 (past the last tile, copies of it, so every wave
        // always has the same number of copies in flight)
        if constexpr (NST > 4) issue_tile(min(3, T - 1), stage(I3{}));
        if constexpr (NST > 5) issue_tile(min(4, T - 1), stage(I4{}));
        if constexpr (NST > 6) issue_tile(min(5, T - 1), stage(I5{}));
        if constexpr (NST > 7) issue_tile(min(6, T - 1), stage(I6{}));
        phase_barrier_lds();                 // tiles 0 .. 2 visible to every wave

        if (grp == 1)
            phase_barrier();                 // group 1 runs one phase behind
        // VALU block -1: K_0's operands
        if (T_w > 0)
            read_k(stage(I0{}));
        phase_barrier_lds();
        for (int t = 0; t < T; t += NST) {
            step(t, I0{});
            if (t + 1 < T) step(t + 1, I1{});
            if (t + 2 < T) step(t + 2, I2{});
            if constexpr (NST > 3) if (t + 3 < T) step(t + 3, I3{});
            if constexpr (NST > 4) if (t + 4 < T) step(t + 4, I4{});
            if constexpr (NST > 5) if (t + 5 < T) step(t + 5, I5{});
            if constexpr (NST > 6) if (t + 6 < T) step(t + 6, I6{});
            if constexpr (NST > 7) if (t + 7 < T) step(t + 7, I7{});
        }
        // the last block: O^T += V_{T-1}^T P_{T-1}^T only
        if (T & 1)
            mfma_block(T, I1{}, stage(I0{}), stage(I0{}), false);
        else
            mfma_block(T, I0{}, stage(I0{}), stage(I0{}), false);
        if (grp == 0)
            phase_barrier();
        wait_vmem();
    }

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

template <int D, int BC, int NST, bool CAUSAL>
hipError_t launch_pp_inst(const FwdArgs &a, hipStream_t s)
{
    const int n_qblk = (a.N + 255) / 256;
    const dim3 grid(a.B * a.H * n_qblk), block(512);
    FwdArgs args = a;
    float c = a.scale * kLog2e;
    void *kargs[] = {&args, &c};
    return hipLaunchKernel((const void *)&fwd_pp_kernel<D, BC, NST, CAUSAL>, grid, block, kargs, 0, s);
}

} // namespace

// LDS stages of the copy ring.  Measured at d = 128 against 4 and 8 stages
// (alternating timings, B1 H16 N16384 to B8 H16 N2048, causal and not): 8 is
// about 1 % slower everywhere, 4 is 2-18 % slower except non-causal
// N = 16384, so 6 (96 KB of LDS).
constexpr int kPpStages = 6;

// two-group forward: d = 64 or 128, 32-key tiles
hipError_t launch_fwd_pp(const FwdArgs &a, int d, bool causal, hipStream_t s)
{
    if (d == 128)
        return causal ? launch_pp_inst<128, 32, kPpStages, true>(a, s)
                      : launch_pp_inst<128, 32, kPpStages, false>(a, s);
    if (d == 64)
        return causal ? launch_pp_inst<64, 32, kPpStages, true>(a, s)
                      : launch_pp_inst<64, 32, kPpStages, false>(a, s);
    return hipErrorInvalidValue;
}

} // namespace fa
