// fa_decode.hip -- decode-shaped forward (a few new query rows against a long
// key/value cache) with the keys split over workgroups, and the merge of the
// splits' partial (O, LSE) results.
//
// The pages single decoding out as the case the training kernels do not fit:
// the cache grows by one token per step and each step is a small, frequent
// product ("Attention" chapter of learn-kernels.com, paragraph on decoding).
// With one query row per (b, h) every key and value byte is used exactly once
// (about one flop per byte), so the kernel is bound by HBM bandwidth and the
// matrix cores have nothing to contribute: it is written as a streaming
// kernel -- coalesced 16-byte loads, fp32 dot products on the vector ALUs,
// row sums across lanes with DPP -- and the key range of each (b, h) is split
// over enough workgroups to keep every CU's loads in flight.  The splits are
// combined with the two-block update of "FlashAttention: Mathematical
// Foundations, IO-Aware Tiling, Online Softmax, and Recomputation Dynamics",
// section "Incremental Online Updates", in log-sum-exp form.
//
// Lane layout (D = 64, 128 or 256): a key row is D/8 lanes wide, each lane owning
// one 16-byte chunk (8 elements); one wave load covers 64/(D/8) consecutive
// rows (1 KB).  Every group of D/8 lanes keeps its own running max, sum and
// output accumulator over the rows it loads; the groups of the workgroup are
// merged through LDS at the end.
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// cache policy of the key/value loads: non-temporal (every byte is read once;
// measured ~15% faster than the default policy for this stream)
constexpr int kNT = 2;

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR lanes (8, 16 or 32, aligned) that hold one key row:
// lane ^ 1, lane ^ 2 (quad permutes), then the mirrored quad of the 8-lane
// half row, then (16 lanes) the mirrored half row, then (32 lanes) the other
// 16-lane row through a lane shuffle.  Every lane of the group ends with the
// full sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float x)
{
    x += dpp<0xB1>(x);      // quad_perm [1, 0, 3, 2]
    x += dpp<0x4E>(x);      // quad_perm [2, 3, 0, 1]
    x += dpp<0x141>(x);     // row_half_mirror
    if constexpr (LPR >= 16)
        x += dpp<0x140>(x); // row_mirror
    if constexpr (LPR == 32)
        x += __shfl_xor(x, 16);
    return x;
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4 &r, float *f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(r[i] << 16);
        f[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
}

// One workgroup (4 waves) per (b, h, split).  NQ >= Nq query rows are kept in
// registers; each wave takes KB-key blocks of the split round-robin.
template <int D, int NQ>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs p)
{
    constexpr int LPR = D / 8;              // lanes per key row
    constexpr int RPI = 64 / LPR;           // key rows per wave load
    constexpr int KB = (NQ >= 4 || D == 256) ? 16 : 32;   // keys per wave step
    constexpr int U = KB / RPI;             // loads per tensor per step
    constexpr int NG = 4 * RPI;             // row groups per workgroup
    constexpr float TAU = 8.0f;             // lazy rescale threshold (log2 units)

    __shared__ float sm_m[NG], sm_l[NG];
    __shared__ __attribute__((aligned(16))) float sm_o[NG][D];

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane / LPR, cc = lane % LPR;
    const int split = blockIdx.x % p.S;
    const int bh = blockIdx.x / p.S;
    const int b = bh / p.H;
    int len = p.kv_lens ? p.kv_lens[b] : p.Nk;
    len = min(max(len, 0), p.Nk);
    const int k0 = split * p.chunk;
    const int k1 = min(k0 + p.chunk, len);
    const float c = p.scale * kLog2e;       // scores in log2 units

    const size_t hoff = (size_t)bh * p.Nk * D;
    const auto rk = head_rsrc((const bf16 *)p.k + hoff, p.Nk, D);
    const auto rv = head_rsrc((const bf16 *)p.v + hoff, p.Nk, D);

    // this lane's 8 elements of each query row, as bf16 pairs
    u32x4 qr[NQ];
    int lim[NQ];        // query t sees keys < lim[t]
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
        qr[t] = t < p.Nq ? *(const u32x4 *)((const bf16 *)p.q + ((size_t)bh * p.Nq + t) * D + 8 * cc)
                         : u32x4{0, 0, 0, 0};
        lim[t] = min(k1, p.causal ? len - p.Nq + t + 1 : len);
    }

    float m[NQ], l[NQ], o[NQ][8];
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
        m[t] = -INFINITY;
        l[t] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[t][e] = 0.0f;
    }

    const unsigned lane_off = (unsigned)((g * D + 8 * cc) * 2);
    auto load = [&](int kb, u32x4 (&kr)[U], u32x4 (&vr)[U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off + (unsigned)(kb + u * RPI) * (unsigned)(D * 2), 0, kNT);
#pragma unroll
        for (int u = 0; u < U; ++u)
            vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off + (unsigned)(kb + u * RPI) * (unsigned)(D * 2), 0, kNT);
    };
    auto step = [&](int kb, const u32x4 (&kr)[U], const u32x4 (&vr)[U]) __attribute__((always_inline)) {
        // scores and probabilities (kept in pr), one query row at a time
        float pr[NQ][U];
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            if (t >= p.Nq)
                break;
            float mb = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // copy the words out first: a bit-cast applied directly to
                    // a vector element reads element 0 whatever the index
                    const unsigned qw = qr[t][i], kw = kr[u][i];
                    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw),
                                                          __builtin_bit_cast(bf16x2, kw), acc, false);
                }
                acc = group_sum<LPR>(acc) * c;
                const int key = kb + u * RPI + g;
                pr[t][u] = key < lim[t] ? acc : -INFINITY;
                mb = fmaxf(mb, pr[t][u]);
            }
            // move the reference max only when this block exceeds it by 2^TAU
            const float mn = mb > m[t] + TAU ? mb : m[t];
            if (__any(mn != m[t])) {
                const float a = mn == m[t] ? 1.0f : exp2_hw(m[t] - mn);
                l[t] *= a;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[t][e] *= a;
                m[t] = mn;
            }
            const float ms = m[t] == -INFINITY ? 0.0f : m[t];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pr[t][u] = exp2_hw(pr[t][u] - ms);
                l[t] += pr[t][u];
            }
        }
        // O += P V, each value chunk converted once for every query row
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[8];
            bf16x8_to_f32(vr[u], vf);
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
                if (t >= p.Nq)
                    break;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[t][e] = fmaf(pr[t][u], vf[e], o[t][e]);
            }
        }
    };

    // Each wave walks its blocks kb, kb + 4 KB, ... with the next block's
    // loads issued before the current block is computed (two register sets
    // used in turn).
    int kb = k0 + wave * KB;
    if (kb < k1) {
        u32x4 ka[U], va[U], kn[U], vn[U];
        load(kb, ka, va);
        for (;;) {
            int nx = kb + 4 * KB;
            if (nx < k1)
                load(nx, kn, vn);
            step(kb, ka, va);
            if (nx >= k1)
                break;
            kb = nx;
            nx = kb + 4 * KB;
            if (nx < k1)
                load(nx, ka, va);
            step(kb, kn, vn);
            if (nx >= k1)
                break;
            kb = nx;
        }
    }

    // merge the NG row groups of the workgroup, one query row at a time
    const int G = wave * RPI + g;
    const size_t R = (size_t)p.B * p.H * p.Nq;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
        if (t >= p.Nq)
            break;
        if (cc == 0) {
            sm_m[G] = m[t];
            sm_l[G] = l[t];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sm_o[G][8 * cc + e] = o[t][e];
        __syncthreads();
        if (threadIdx.x < D) {
            const int e = threadIdx.x;
            float M = -INFINITY;
#pragma unroll
            for (int i = 0; i < NG; ++i)
                M = fmaxf(M, sm_m[i]);
            float L = 0.0f, acc = 0.0f;
            if (M != -INFINITY) {
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    const float w = sm_m[i] == -INFINITY ? 0.0f : exp2_hw(sm_m[i] - M);
                    L = fmaf(sm_l[i], w, L);
                    acc = fmaf(sm_o[i][e], w, acc);
                }
            }
            const float out = L > 0.0f ? acc / L : 0.0f;
            const float lse = L > 0.0f ? kLn2 * (M + __log2f(L)) : -INFINITY;
            const size_t row = (size_t)bh * p.Nq + t;
            if (p.S == 1) {
                ((bf16 *)p.o)[row * D + e] = (bf16)out;
                if (e == 0)
                    p.lse[row] = lse;
            } else {
                p.o_part[((size_t)split * R + row) * D + e] = out;
                if (e == 0)
                    p.lse_part[(size_t)split * R + row] = lse;
            }
        }
        __syncthreads();
    }
}

// One thread per output element: o = sum_s exp(lse_s - lse) o_s with
// lse = log sum_s exp(lse_s).  The S log-sum-exps of a row are read by every
// thread of the row (cache hits after the first).
__global__ __launch_bounds__(256) void merge_kernel(const float *o_parts, const float *lse_parts,
                                                    int S, int R, int d, void *o, float *lse,
                                                    int out_bf16)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)R * d)
        return;
    const int row = (int)(idx / d), e = (int)(idx % d);
    float M = -INFINITY;
    for (int s = 0; s < S; ++s)
        M = fmaxf(M, lse_parts[(size_t)s * R + row]);
    float W = 0.0f, acc = 0.0f;
    if (M != -INFINITY) {
#pragma unroll 4
        for (int s = 0; s < S; ++s) {
            const float x = lse_parts[(size_t)s * R + row];
            const float w = x == -INFINITY ? 0.0f : __expf(x - M);
            const float v = o_parts[((size_t)s * R + row) * d + e];
            W += w;
            acc = w == 0.0f ? acc : fmaf(w, v, acc);
        }
    }
    const float out = W > 0.0f ? acc / W : 0.0f;
    if (out_bf16)
        ((bf16 *)o)[idx] = (bf16)out;
    else
        ((float *)o)[idx] = out;
    if (e == 0)
        lse[row] = W > 0.0f ? M + __logf(W) : -INFINITY;
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(a.B * a.H * a.S)), block(256);
    if (a.Nq <= 1)
        decode_kernel<D, 1><<<grid, block, 0, s>>>(a);
    else if (a.Nq <= 2)
        decode_kernel<D, 2><<<grid, block, 0, s>>>(a);
    else if (a.Nq <= 4)
        decode_kernel<D, 4><<<grid, block, 0, s>>>(a);
    else
        decode_kernel<D, 8><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t s)
{
    if (d == 64)
        return launch_decode_d<64>(a, s);
    if (d == 128)
        return launch_decode_d<128>(a, s);
    return launch_decode_d<256>(a, s);
}

hipError_t launch_merge(const float *o_parts, const float *lse_parts, int S, int R, int d, void *o,
                        float *lse, bool out_bf16, hipStream_t s)
{
    const int64_t n = (int64_t)R * d;
    merge_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(o_parts, lse_parts, S, R, d,
                                                                        o, lse, out_bf16 ? 1 : 0);
    return hipGetLastError();
}

} // namespace fa
