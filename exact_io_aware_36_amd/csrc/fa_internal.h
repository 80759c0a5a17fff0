// fa_internal.h -- shared declarations between the C-ABI layer and the
// kernel translation units of libfa.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a forward launch needs.  Tensors are dense [B][H][N][D].
struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, H, N;
    float scale;            // softmax scale (natural units)
    const int32_t *kv_lens; // nullable device int32[B]
    const uint8_t *mask;    // block mask (sparse launches only)
    int nb;                 // mask blocks per side (sparse launches only)
    int wg_slots = 0;       // workgroups resident at once per XCD (causal order; 0 = unknown)
};

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *dvec;            // workspace: D_i = dO_i . O_i, fp32 [B][H][N]
    float *lse2;            // workspace: LSE_i * log2(e) (+inf where LSE = -inf)
    int B, H, N;
    float scale;
    const int32_t *kv_lens;
    const uint8_t *mask;    // block mask (sparse launches only)
    int nb;                 // mask blocks per side (sparse launches only)
    int tile_q = 0;         // query rows per tile of the dK/dV kernel (0 = 64; 64 or 128)
};

// Kernel launchers; each returns the launch status and enqueues only.
hipError_t launch_fwd_bf16(const FwdArgs &a, int d, int tile_n, bool causal, bool sparse,
                           hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs &a, int d, bool causal, hipStream_t s);
// the two-group forward (fa_fwd_pp.hip): d = 64 or 128, 32-key tiles, dense
hipError_t launch_fwd_pp(const FwdArgs &a, int d, bool causal, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs &a, int d, bool causal, bool sparse, hipStream_t s);
enum class BwdStage { Dot, DkDv, Dq };
// the dK, dV launch(es) of the backward (fa_bwd_dkdv.hip)
hipError_t launch_bwd_dkdv(const BwdArgs &a, int d, bool causal, bool sparse, hipStream_t s);
hipError_t launch_bwd_stage(const BwdArgs &a, int d, bool causal, bool sparse, BwdStage stage,
                            hipStream_t s);

// Decode-shaped forward with the keys split over workgroups.  q and o are
// [B][H][Nq][D], k and v [B][H][Nk][D].  Split s covers keys
// [s*chunk, (s+1)*chunk); with S == 1 the kernel writes o and lse directly,
// otherwise each split writes its own normalised output and log-sum-exp to
// o_part [S][B*H*Nq][D] and lse_part [S][B*H*Nq] for the merge kernel.
struct DecodeArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    float *o_part, *lse_part;
    int B, H, Nq, Nk, S, chunk;
    float scale;
    const int32_t *kv_lens;  // nullable device int32[B]
    int causal;
};
hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t s);

// Merge of S partial results per row: o_parts [S][R][d] fp32 (each part
// normalised), lse_parts [S][R] (natural log, -inf = empty part) into o [R][d]
// (bf16 when out_bf16, else fp32) and lse [R].
hipError_t launch_merge(const float *o_parts, const float *lse_parts, int S, int R, int d,
                        void *o, float *lse, bool out_bf16, hipStream_t s);

// FP8 (E4M3) quantiser: per 128-row block (per_head = false) or one scale per
// (b, h) (per_head = true, amax_ws [B][H][ceil(N/128)] scratch); signs
// (nullable) applies the random-sign Hadamard rotation; transpose writes
// [B][H][d][N].
hipError_t launch_quant_fp8(const void *x, void *x8, float *descale, float *amax_ws,
                            const float *signs, int B, int H, int N, int d, bool per_head,
                            bool transpose, hipStream_t s);
// FP8 forward: q8, k8 [B][H][N][d] E4M3, v8t [B][H][d][N] E4M3; qs, ks
// [B][H][ceil(N/128)] descales, vs [B][H]; o bf16, lse fp32.
hipError_t launch_fwd_fp8(const void *q8, const void *k8, const void *v8t, const float *qs,
                          const float *ks, const float *vs, void *o, float *lse, int B, int H,
                          int N, int d, bool causal, float scale, const int32_t *kv_lens,
                          hipStream_t s);

constexpr int MAX_MASK_BLOCKS = 512;   // block-sparse: N <= 65536 with 128-blocks

// Wave 0 of the workgroup lists, in increasing order, the indices i < n with
// mask[i * stride] != 0 into list[] (LDS) and their count into *count; the
// caller synchronises the workgroup before reading them.
__device__ __forceinline__ void list_nonzero(const uint8_t *mask, int n, int stride, int *list,
                                             int *count)
{
    const int lane = threadIdx.x & 63;
    int cnt = 0;
    for (int base = 0; base < n; base += 64) {
        const int i = base + lane;
        const bool on = i < n && mask[(size_t)i * stride] != 0;
        const unsigned long long bits = __ballot(on);
        const int pos = cnt + __popcll(bits & ((1ull << lane) - 1ull));
        if (on)
            list[pos] = i;
        cnt += __popcll(bits);
    }
    if (lane == 0)
        *count = cnt;
}

// The workgroup-to-tile remap used by every attention grid: workgroups are
// dispatched round-robin over the 8 XCDs, so work item w is given to the
// workgroup that lands on XCD (w / per_xcd); consecutive work items then share
// one XCD's L2.  Falls back to the identity when total % 8 != 0.
__device__ __forceinline__ int xcd_remap(int bid, int total)
{
    constexpr int NXCD = 8;
    if (total % NXCD != 0)
        return bid;
    const int per_xcd = total / NXCD;
    return (bid % NXCD) * per_xcd + bid / NXCD;
}

// Work item of a causal grid of n_bh heads (b * H + h) times nblk row blocks
// whose work falls with the block's rank: sets bh and rank, rank 0 being the
// block with the most work.  Each XCD owns whole heads, as with xcd_remap,
// and takes them in groups of `group` heads; within a group the heads are
// interleaved in decreasing work (its r-th item is rank r / gs of the group's
// head r % gs), so the XCD runs longest-first across the group.  Head by head
// (group = 1, xcd_remap's order) a later head's longest blocks start after an
// earlier head's shortest ones and set the finish time; interleaving every
// head of the XCD instead keeps all of their tiles in use at once, which
// overflows the XCD's L2 and multiplies the L2 misses.  The group size is
// chosen so the group's streamed tiles fit the L2 (l2_group); heads of
// fewer than four blocks keep the head-major order.
__device__ __forceinline__ void causal_item(int bid, int n_bh, int nblk, int group, int &bh,
                                            int &rank)
{
    constexpr int NXCD = 8;
    if (n_bh % NXCD == 0) {
        const int hp = n_bh / NXCD;                  // heads per XCD
        const int r = bid / NXCD;                    // dispatch rank within the XCD
        // with under four blocks per head the blocks' work differs little and
        // head-major order measured faster (B64 H16 N256 d128: 0.062 against
        // 0.069 ms for the forward)
        const int g = nblk < 4 ? 1 : min(max(group, 1), hp);
        const int h0 = r / (g * nblk) * g;           // first head of r's group
        const int gs = min(g, hp - h0);              // heads in that group
        const int rr = r - h0 * nblk;
        bh = (bid % NXCD) * hp + h0 + rr % gs;
        rank = rr / gs;
    } else {
        const int w = xcd_remap(bid, n_bh * nblk);
        bh = w / nblk;
        rank = w % nblk;
    }
}

// Rotation of a causal grid's rank order (causal_item) for one case: when an
// XCD's heads form a single group and its items exceed one round of resident
// workgroups (slots_per_xcd) by part of a round, the ranks that would start
// last -- the shortest rows, which then run nearly alone and are bound by
// their start-up latency -- are moved to the front, so that they run beside
// the first round's long blocks.  Returns the number of ranks to move to the
// front (0: keep the longest-first order).  Measured on the forward at
// B8 H16 N1024 d64 causal: 30.6 -> 29.2 us with two ranks moved.
__device__ __forceinline__ int causal_rotation(int n_bh, int nblk, int group, int slots_per_xcd)
{
    constexpr int NXCD = 8;
    if (slots_per_xcd <= 0 || n_bh % NXCD != 0 || nblk < 4)
        return 0;
    const int hp = n_bh / NXCD;
    if (min(max(group, 1), hp) != hp)
        return 0;                                // several groups per XCD: order kept
    const int k = nblk - slots_per_xcd / hp;     // ranks that do not start in the first round
    return (k > 0 && k < nblk) ? k : 0;
}

// Heads whose streamed [N][D] tensors (bytes_per_row bytes per row and head,
// e.g. K and V in bf16: 4 D) fit one XCD's 4 MB L2 together; at least 1.
__device__ __forceinline__ int l2_group(int N, int bytes_per_row)
{
    const unsigned long long per_head = (unsigned long long)N * (unsigned long long)bytes_per_row;
    const unsigned long long g = (4ull << 20) / (per_head > 0 ? per_head : 1);
    return g < 1 ? 1 : (g > 1024 ? 1024 : (int)g);
}

} // namespace fa
