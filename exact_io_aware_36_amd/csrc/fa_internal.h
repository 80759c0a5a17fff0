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
};

// Kernel launchers; each returns the launch status and enqueues only.
hipError_t launch_fwd_bf16(const FwdArgs &a, int d, int tile_n, bool causal, bool sparse,
                           hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs &a, int d, bool causal, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs &a, int d, bool causal, hipStream_t s);
enum class BwdStage { Dot, DkDv, Dq };
hipError_t launch_bwd_stage(const BwdArgs &a, int d, bool causal, BwdStage stage, hipStream_t s);

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

} // namespace fa
