// fa_kvouter.h -- launch interface of the key/value-outer forward (the IO
// ablation of the loop order, fa_kvouter.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// fp32 O accumulator [B][H][N][D] and running statistics m (log2 units), l
// [B][H][N] live in the caller's workspace between the launches.
struct KvOuterArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    float *o_acc, *m, *l;
    int B, H, N;
    float scale;
};
hipError_t launch_fwd_kvouter(const KvOuterArgs &a, int d, bool causal, hipStream_t s);

} // namespace fa
