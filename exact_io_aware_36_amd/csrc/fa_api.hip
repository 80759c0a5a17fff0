// fa_api.hip -- the C ABI of libfa.so: argument checks, kernel choice and
// launch.  Every entry point only enqueues on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_internal.h"
#include "fa_kvouter.h"

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// d = 256 is built for the bf16 paths (forward, backward, block-sparse)
fa_status check_common(const void *q, const void *k, const void *v, int B, int H, int N, int d,
                       float scale, bool allow_256 = false)
{
    if (!q || !k || !v)
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1)
        return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale))
        return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128 && !(allow_256 && d == 256))
        return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * H * N * d >= ((int64_t)1 << 31))
        return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

} // namespace

extern "C" {

const char *fa_status_str(fa_status s)
{
    switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH";
    }
    return "FA_ERR_UNKNOWN";
}

fa_status fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                    int H, int N, int d, int causal, float scale, const int32_t *kv_lens,
                    fa_dtype dtype, int tile_n, fa_stream_t stream)
{
    fa_status st = check_common(q, k, v, B, H, N, d, scale, dtype == FA_DTYPE_BF16);
    if (st != FA_OK)
        return st;
    if (!o || !lse || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;
    if (kv_lens && !aligned(kv_lens, 4))
        return FA_ERR_INVALID_ARG;
    fa::FwdArgs a{q, k, v, o, lse, B, H, N, scale, kv_lens, nullptr, 0};
    hipStream_t s = (hipStream_t)stream;
    if (dtype == FA_DTYPE_BF16) {
        // key tiles: 32, 64, 128 or 256 at d = 64, 128; 32 or 64 at d = 256 (LDS)
        const bool ok = d == 256 ? (tile_n == 0 || tile_n == 32 || tile_n == 64)
                                 : (tile_n == 0 || tile_n == 32 || tile_n == 64 || tile_n == 128 ||
                                    tile_n == 256);
        if (!ok)
            return FA_ERR_UNSUPPORTED;
        // default: the two-group kernel (32-key tiles) at d = 128 from
        // N = 2048 on; below that, and at d = 64, the 64-key kernel measured
        // faster (it has twice the workgroups, 128 query rows each)
        if (tile_n == 0)
            tile_n = (d == 128 && N >= 2048) ? 32 : 64;
        if (d != 256 && tile_n == 32)
            return from_hip(fa::launch_fwd_pp(a, d, causal != 0, s));
        return from_hip(fa::launch_fwd_bf16(a, d, tile_n, causal != 0, false, s));
    }
    if (dtype == FA_DTYPE_FP32) {
        if (tile_n != 0 && tile_n != 32)
            return FA_ERR_UNSUPPORTED;
        return from_hip(fa::launch_fwd_f32(a, d, causal != 0, s));
    }
    return FA_ERR_UNSUPPORTED;
}

fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                 int N, int d, int causal, float scale, const int32_t *kv_lens, fa_dtype dtype,
                 fa_stream_t stream)
{
    return fa_fwd_ex(q, k, v, o, lse, B, H, N, d, causal, scale, kv_lens, dtype, 0, stream);
}

// workspace: D then LSE * log2(e), each fp32 [B][H][N] rounded up to 256 B
static size_t ws_region(int B, int H, int N) { return ((size_t)B * H * N * sizeof(float) + 255) / 256 * 256; }

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d)
{
    if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128 && d != 256))
        return 0;
    return 2 * ws_region(B, H, N);
}

// Shared checks of fa_bwd and its stages.  A stage that does not use one of
// the tensors passes one it does use in its place.
static fa_status check_bwd(const void *q, const void *k, const void *v, const void *o,
                           const void *dout, const float *lse, const void *dq, const void *dk,
                           const void *dv, int B, int H, int N, int d, float scale,
                           const int32_t *kv_lens, fa_dtype dtype, const void *workspace,
                           size_t workspace_bytes)
{
    fa_status st = check_common(q, k, v, B, H, N, d, scale, dtype == FA_DTYPE_BF16);
    if (st != FA_OK)
        return st;
    if (!o || !dout || !lse || !dq || !dk || !dv)
        return FA_ERR_INVALID_ARG;
    if (!aligned(o, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) ||
        !aligned(dv, 16) || !aligned(lse, 4) || (kv_lens && !aligned(kv_lens, 4)))
        return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    const size_t need = fa_bwd_workspace_bytes(B, H, N, d);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return FA_ERR_WORKSPACE;
    return FA_OK;
}

fa_status fa_bwd_ex(const void *q, const void *k, const void *v, const void *o, const void *dout,
                    const float *lse, void *dq, void *dk, void *dv, int B, int H, int N, int d,
                    int causal, float scale, const int32_t *kv_lens, fa_dtype dtype, int tile_n,
                    void *workspace, size_t workspace_bytes, fa_stream_t stream)
{
    fa_status st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, kv_lens, dtype,
                             workspace, workspace_bytes);
    if (st != FA_OK)
        return st;
    // query rows per tile of the dK/dV kernel: 64, or 128 at d <= 128
    if (!(tile_n == 0 || tile_n == 64 || (tile_n == 128 && d != 256)))
        return FA_ERR_UNSUPPORTED;
    float *ws = (float *)workspace;
    float *ws2 = (float *)((char *)workspace + ws_region(B, H, N));
    fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, ws, ws2, B, H, N, scale, kv_lens};
    a.tile_q = tile_n;
    return from_hip(fa::launch_bwd_bf16(a, d, causal != 0, false, (hipStream_t)stream));
}

fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, void *dq, void *dk, void *dv, int B, int H, int N, int d,
                 int causal, float scale, const int32_t *kv_lens, fa_dtype dtype,
                 void *workspace, size_t workspace_bytes, fa_stream_t stream)
{
    fa_status st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, kv_lens, dtype,
                             workspace, workspace_bytes);
    if (st != FA_OK)
        return st;
    float *ws = (float *)workspace;
    float *ws2 = (float *)((char *)workspace + ws_region(B, H, N));
    fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, ws, ws2, B, H, N, scale, kv_lens};
    return from_hip(fa::launch_bwd_bf16(a, d, causal != 0, false, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// The backward without caller workspace.  Its scratch (D, then LSE * log2(e),
// fp32, one value per query row each) lives in this file-scope device array:
// every GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` only names the symbol; its device address comes
// from hipGetSymbolAddress, once per device, kept in scratch_ptr[].
constexpr int kNoAllocMaxRows = 1 << 20;     // B * H * N limit: 8 MiB of scratch
static __device__ __align__(256) float scratch[2 * kNoAllocMaxRows];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float *scratch_ptr[kMaxDevices];

// device address of `scratch` on the current device (looked up on the
// device's first call)
hipError_t scratch_on_current_device(float **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        scratch_ptr[dev] = (float *)p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}
} // namespace

int fa_bwd_noalloc_max_rows(void) { return kNoAllocMaxRows; }

fa_status fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                         const void *dout, const float *lse, void *dq, void *dk, void *dv, int B,
                         int H, int N, int d, int causal, float scale, const int32_t *kv_lens,
                         fa_dtype dtype, fa_stream_t stream)
{
    // the argument checks of fa_bwd, with a stand-in workspace of the size
    // it requires (none is read)
    const size_t need = fa_bwd_workspace_bytes(B, H, N, d);
    fa_status st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, kv_lens, dtype,
                             (const void *)256, need);
    if (st != FA_OK)
        return st;
    if ((int64_t)B * H * N > kNoAllocMaxRows)
        return FA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (s) {   // the stream must belong to the current device, whose scratch is used
        int cur = -1, sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(s, &sdev) != hipSuccess)
            return FA_ERR_LAUNCH;
        if (cur != sdev)
            return FA_ERR_INVALID_ARG;
    }
    float *ws = nullptr;
    if (scratch_on_current_device(&ws) != hipSuccess)
        return FA_ERR_LAUNCH;
    // D in the first half, LSE * log2(e) in the second; every row the kernels
    // read is written by the preprocessing kernel first, so nothing is cleared
    fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, ws, ws + kNoAllocMaxRows, B, H, N, scale,
                  kv_lens};
    return from_hip(fa::launch_bwd_bf16(a, d, causal != 0, false, s));
}

fa_status fa_bwd_preprocess(const void *o, const void *dout, const float *lse, int B, int H,
                            int N, int d, fa_dtype dtype, void *workspace, size_t workspace_bytes,
                            fa_stream_t stream)
{
    // o and dout stand in for every other tensor pointer of the full check
    fa_status st = check_bwd(o, o, o, o, dout, lse, o, o, o, B, H, N, d, 1.f, nullptr, dtype,
                             workspace, workspace_bytes);
    if (st != FA_OK)
        return st;
    float *ws = (float *)workspace;
    float *ws2 = (float *)((char *)workspace + ws_region(B, H, N));
    fa::BwdArgs a{nullptr, nullptr, nullptr, o, dout, lse, nullptr, nullptr, nullptr, ws, ws2,
                  B, H, N, 1.f, nullptr};
    return from_hip(fa::launch_bwd_stage(a, d, false, false, fa::BwdStage::Dot, (hipStream_t)stream));
}

fa_status fa_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout,
                      const float *lse, void *dk, void *dv, int B, int H, int N, int d,
                      int causal, float scale, const int32_t *kv_lens, fa_dtype dtype,
                      const void *workspace, size_t workspace_bytes, fa_stream_t stream)
{
    fa_status st = check_bwd(q, k, v, dout, dout, lse, dk, dk, dv, B, H, N, d, scale, kv_lens,
                             dtype, workspace, workspace_bytes);
    if (st != FA_OK)
        return st;
    float *ws = (float *)workspace;
    float *ws2 = (float *)((char *)workspace + ws_region(B, H, N));
    fa::BwdArgs a{q, k, v, nullptr, dout, lse, nullptr, dk, dv, ws, ws2, B, H, N, scale, kv_lens};
    return from_hip(fa::launch_bwd_stage(a, d, causal != 0, false, fa::BwdStage::DkDv, (hipStream_t)stream));
}

fa_status fa_bwd_dq(const void *q, const void *k, const void *v, const void *dout,
                    const float *lse, void *dq, int B, int H, int N, int d, int causal,
                    float scale, const int32_t *kv_lens, fa_dtype dtype, const void *workspace,
                    size_t workspace_bytes, fa_stream_t stream)
{
    fa_status st = check_bwd(q, k, v, dout, dout, lse, dq, dq, dq, B, H, N, d, scale, kv_lens,
                             dtype, workspace, workspace_bytes);
    if (st != FA_OK)
        return st;
    float *ws = (float *)workspace;
    float *ws2 = (float *)((char *)workspace + ws_region(B, H, N));
    fa::BwdArgs a{q, k, v, nullptr, dout, lse, dq, nullptr, nullptr, ws, ws2, B, H, N, scale,
                  kv_lens};
    return from_hip(fa::launch_bwd_stage(a, d, causal != 0, false, fa::BwdStage::Dq, (hipStream_t)stream));
}

fa_status fa_fwd_blocksparse(const void *q, const void *k, const void *v, void *o, float *lse,
                             int B, int H, int N, int d, float scale, const uint8_t *block_mask,
                             int mask_block, fa_dtype dtype, fa_stream_t stream)
{
    fa_status st = check_common(q, k, v, B, H, N, d, scale, dtype == FA_DTYPE_BF16);
    if (st != FA_OK)
        return st;
    if (!o || !lse || !block_mask || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;
    if (mask_block != 128 || N % mask_block != 0)
        return FA_ERR_INVALID_ARG;
    if (N / mask_block > fa::MAX_MASK_BLOCKS)
        return FA_ERR_UNSUPPORTED;
    if (dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    fa::FwdArgs a{q, k, v, o, lse, B, H, N, scale, nullptr, block_mask, N / mask_block};
    return from_hip(fa::launch_fwd_bf16(a, d, 0, false, true, (hipStream_t)stream));
}

fa_status fa_bwd_blocksparse(const void *q, const void *k, const void *v, const void *o,
                             const void *dout, const float *lse, void *dq, void *dk, void *dv,
                             int B, int H, int N, int d, float scale, const uint8_t *block_mask,
                             int mask_block, fa_dtype dtype, void *workspace,
                             size_t workspace_bytes, fa_stream_t stream)
{
    fa_status st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, nullptr, dtype,
                             workspace, workspace_bytes);
    if (st != FA_OK)
        return st;
    if (!block_mask || mask_block != 128 || N % mask_block != 0)
        return FA_ERR_INVALID_ARG;
    if (N / mask_block > fa::MAX_MASK_BLOCKS)
        return FA_ERR_UNSUPPORTED;
    float *ws = (float *)workspace;
    float *ws2 = (float *)((char *)workspace + ws_region(B, H, N));
    fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, ws, ws2, B, H, N, scale, nullptr,
                  block_mask, N / mask_block};
    return from_hip(fa::launch_bwd_bf16(a, d, false, true, (hipStream_t)stream));
}

// Split plan of the split-KV forward: chunk keys per split (a multiple of
// 32), S = ceil(Nk / chunk) splits.  The default aims at 512 workgroups --
// two per CU of the 256, which is what stays resident at the kernel's
// register use, so the whole grid runs in one round -- with at least 256 keys
// per split.
static const int kMaxSplits = 1024;
static void splitkv_plan(int B, int H, int Nk, int num_splits, int *S, int *chunk)
{
    int64_t s = num_splits;
    if (s <= 0) {
        const int64_t bh = (int64_t)B * H;
        s = (512 + bh - 1) / bh;
        s = s < (Nk + 255) / 256 ? s : (Nk + 255) / 256;
    }
    s = s < (Nk + 31) / 32 ? s : (Nk + 31) / 32;
    s = s < kMaxSplits ? s : kMaxSplits;
    s = s < 1 ? 1 : s;
    const int ch = (int)(((Nk + s - 1) / s + 31) / 32 * 32);
    *chunk = ch;
    *S = (Nk + ch - 1) / ch;
}

int fa_splitkv_splits(int B, int H, int Nk, int num_splits)
{
    if (B < 1 || H < 1 || Nk < 1 || num_splits < 0)
        return 0;
    int S, chunk;
    splitkv_plan(B, H, Nk, num_splits, &S, &chunk);
    return S;
}

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits)
{
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || num_splits < 0 || (d != 64 && d != 128 && d != 256))
        return 0;
    int S, chunk;
    splitkv_plan(B, H, Nk, num_splits, &S, &chunk);
    if (S == 1)
        return 0;
    const size_t R = (size_t)B * H * Nq;
    return round256((size_t)S * R * d * sizeof(float)) + round256((size_t)S * R * sizeof(float));
}

fa_status fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                         int B, int H, int Nq, int Nk, int d, int causal, float scale,
                         const int32_t *kv_lens, int num_splits, fa_dtype dtype,
                         void *workspace, size_t workspace_bytes, fa_stream_t stream)
{
    if (!q || !k || !v || !o || !lse)
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || num_splits < 0)
        return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale))
        return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128 && d != 256)
        return FA_ERR_UNSUPPORTED;
    const int64_t nmax = Nq > Nk ? Nq : Nk;
    if ((int64_t)B * H * nmax * d >= ((int64_t)1 << 31))
        return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4) || (kv_lens && !aligned(kv_lens, 4)))
        return FA_ERR_INVALID_ARG;
    if (Nq > 8 || dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    int S, chunk;
    splitkv_plan(B, H, Nk, num_splits, &S, &chunk);
    const size_t need = fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return FA_ERR_WORKSPACE;
    const size_t R = (size_t)B * H * Nq;
    float *o_part = (float *)workspace;
    float *lse_part = S > 1 ? (float *)((char *)workspace + round256((size_t)S * R * d * sizeof(float)))
                            : nullptr;
    fa::DecodeArgs a{q, k, v, o, lse, o_part, lse_part, B, H, Nq, Nk, S, chunk, scale, kv_lens,
                     causal != 0};
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = fa::launch_decode(a, d, s);
    if (e != hipSuccess || S == 1)
        return from_hip(e);
    return from_hip(fa::launch_merge(o_part, lse_part, S, (int)R, d, o, lse, true, s));
}

fa_status fa_merge(const float *o_parts, const float *lse_parts, int S, int R, int d, void *o,
                   float *lse, fa_dtype dtype, fa_stream_t stream)
{
    if (!o_parts || !lse_parts || !o || !lse)
        return FA_ERR_INVALID_ARG;
    if (S < 1 || R < 1 || d < 1 || d > 1024 || (int64_t)R * d >= ((int64_t)1 << 31))
        return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP32)
        return FA_ERR_UNSUPPORTED;
    if (!aligned(o_parts, 4) || !aligned(lse_parts, 4) || !aligned(lse, 4) ||
        !aligned(o, dtype == FA_DTYPE_BF16 ? 2 : 4))
        return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_merge(o_parts, lse_parts, S, R, d, o, lse, dtype == FA_DTYPE_BF16,
                                     (hipStream_t)stream));
}

size_t fa_quantize_fp8_workspace_bytes(int B, int H, int N, int d, int block_rows)
{
    if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128) || block_rows != 0)
        return 0;
    return round256((size_t)B * H * ((N + 127) / 128) * sizeof(float));
}

fa_status fa_quantize_fp8(const void *x, void *x8, float *descale, int B, int H, int N, int d,
                          int block_rows, const float *signs, int transpose, void *workspace,
                          size_t workspace_bytes, fa_stream_t stream)
{
    if (!x || !x8 || !descale)
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || (block_rows != 0 && block_rows != 128))
        return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128)
        return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * H * N * d >= ((int64_t)1 << 31) || (transpose && N % 16 != 0))
        return FA_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(descale, 4) || (signs && !aligned(signs, 4)))
        return FA_ERR_INVALID_ARG;
    const size_t need = fa_quantize_fp8_workspace_bytes(B, H, N, d, block_rows);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return FA_ERR_WORKSPACE;
    return from_hip(fa::launch_quant_fp8(x, x8, descale, (float *)workspace, signs, B, H, N, d,
                                         block_rows == 0, transpose != 0, (hipStream_t)stream));
}

fa_status fa_fwd_fp8(const void *q8, const void *k8, const void *v8t, const float *q_descale,
                     const float *k_descale, const float *v_descale, void *o, float *lse, int B,
                     int H, int N, int d, int causal, float scale, const int32_t *kv_lens,
                     fa_stream_t stream)
{
    if (!q8 || !k8 || !v8t || !q_descale || !k_descale || !v_descale || !o || !lse)
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || N % 16 != 0)
        return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale))
        return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128)
        return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * H * N * d >= ((int64_t)1 << 31))
        return FA_ERR_INVALID_ARG;
    if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8t, 16) || !aligned(o, 16) ||
        !aligned(q_descale, 4) || !aligned(k_descale, 4) || !aligned(v_descale, 4) ||
        !aligned(lse, 4) || (kv_lens && !aligned(kv_lens, 4)))
        return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_fwd_fp8(q8, k8, v8t, q_descale, k_descale, v_descale, o, lse, B, H,
                                       N, d, causal != 0, scale, kv_lens, (hipStream_t)stream));
}

// Key/value-outer forward (the IO ablation).  Workspace: fp32 O accumulator
// [B][H][N][d], then m and l fp32 [B][H][N], each rounded up to 256 B.
size_t fa_fwd_kvouter_workspace_bytes(int B, int H, int N, int d)
{
    if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128))
        return 0;
    if ((int64_t)B * H * N * d >= ((int64_t)1 << 31))
        return 0;
    return ((size_t)B * H * N * d * sizeof(float) + 255) / 256 * 256 + 2 * ws_region(B, H, N);
}

fa_status fa_fwd_kvouter(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                         int H, int N, int d, int causal, float scale, void *workspace,
                         size_t workspace_bytes, fa_stream_t stream)
{
    fa_status st = check_common(q, k, v, B, H, N, d, scale);
    if (st != FA_OK)
        return st;
    if (!o || !lse || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;
    const size_t need = fa_fwd_kvouter_workspace_bytes(B, H, N, d);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return FA_ERR_WORKSPACE;
    float *o_acc = (float *)workspace;
    float *m = (float *)((char *)workspace + ((size_t)B * H * N * d * sizeof(float) + 255) / 256 * 256);
    float *l = (float *)((char *)m + ws_region(B, H, N));
    fa::KvOuterArgs a{q, k, v, o, lse, o_acc, m, l, B, H, N, scale};
    return from_hip(fa::launch_fwd_kvouter(a, d, causal != 0, (hipStream_t)stream));
}

} // extern "C"
