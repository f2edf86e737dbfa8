// token_reduction.hip -- merge paired rows of the residual stream and restore
// the full-resolution rows from the bypass.
//
// Page "MiniMax H3 Inference Engine voor Mac computers", presets and
// implementation notes: the token-reduction mode pairs adjacent horizontal
// target-video tokens after block 3, keeps text, audio and reference tokens
// exact, and restores the full-resolution state, kept as a bypass, before a
// later block.  Readings: a pair merges to the mean of its two rows; the
// restore gives both rows the bypass plus the change the reduced blocks made
// to their merged row.
//
// HBM-bound: one 256-thread block per reduced row, 16-byte chunks, fp32
// arithmetic, one bf16 rounding per output.  merge reads 1-2 rows and writes
// one; restore reads the two reduced rows and 1-2 bypass rows and writes
// 1-2 rows.
#include "internal.h"

#include <algorithm>

namespace pma {
namespace {

__device__ __forceinline__ void unpack8(const u16x8 r, float *f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = bf16_bits_to_f32(r[e]);
}

__device__ __forceinline__ uint4 pack8(const float *f) {
    uint4 w;
    w.x = pack_bf16x2(f[0], f[1]);
    w.y = pack_bf16x2(f[2], f[3]);
    w.z = pack_bf16x2(f[4], f[5]);
    w.w = pack_bf16x2(f[6], f[7]);
    return w;
}

__global__ __launch_bounds__(256) void token_merge_kernel(TokenLaunch a) {
    const int i = blockIdx.x;
    const int r0 = a.src0[i], r1 = a.src1[i];
    uint16_t *dst = a.xr_out + (int64_t)i * a.hidden;
    const bool ok0 = (uint32_t)r0 < (uint32_t)a.L;
    const bool pair = (uint32_t)r1 < (uint32_t)a.L;
    if (!ok0) {
        // an entry outside the sequence (pma_token_plan_check reports it):
        // the reduced row is written as zeros rather than left stale
        for (int c = 8 * threadIdx.x; c < a.hidden; c += 8 * 256)
            *reinterpret_cast<uint4 *>(dst + c) = make_uint4(0, 0, 0, 0);
        return;
    }
    const uint16_t *x0 = a.x + (int64_t)r0 * a.hidden;
    const uint16_t *x1 = a.x + (int64_t)(pair ? r1 : r0) * a.hidden;
    for (int c = 8 * threadIdx.x; c < a.hidden; c += 8 * 256) {
        float f0[8], f1[8], m[8];
        unpack8(*reinterpret_cast<const u16x8 *>(x0 + c), f0);
        unpack8(*reinterpret_cast<const u16x8 *>(x1 + c), f1);
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = pair ? (f0[e] + f1[e]) * 0.5f : f0[e];
        *reinterpret_cast<uint4 *>(dst + c) = pack8(m);
    }
}

__global__ __launch_bounds__(256) void token_restore_kernel(TokenLaunch a) {
    const int i = blockIdx.x;
    const int r0 = a.src0[i], r1 = a.src1[i];
    const bool ok0 = (uint32_t)r0 < (uint32_t)a.L;
    const bool pair = (uint32_t)r1 < (uint32_t)a.L;
    const uint16_t *before = a.xr_before + (int64_t)i * a.hidden;
    const uint16_t *after = a.xr_in + (int64_t)i * a.hidden;
    for (int c = 8 * threadIdx.x; c < a.hidden; c += 8 * 256) {
        float fb[8], fa[8], d[8];
        unpack8(*reinterpret_cast<const u16x8 *>(before + c), fb);
        unpack8(*reinterpret_cast<const u16x8 *>(after + c), fa);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = fa[e] - fb[e];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = k ? r1 : r0;
            if (!(k ? pair : ok0)) continue;
            float fx[8];
            unpack8(*reinterpret_cast<const u16x8 *>(a.x + (int64_t)r * a.hidden + c), fx);
#pragma unroll
            for (int e = 0; e < 8; ++e) fx[e] += d[e];
            *reinterpret_cast<uint4 *>(a.x_out + (int64_t)r * a.hidden + c) = pack8(fx);
        }
    }
}

// ---- plan check.  ws: [0] status bits, [1] first bad entry, [2] first full
// row named by no entry or by several, [3 .. 3 + L) how often each full row
// is named.  Cleared by a kernel (no memset), so the sequence can be captured.
__global__ __launch_bounds__(256) void token_plan_clear_kernel(int32_t *ws, int32_t L) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < (int64_t)L + 3;
         i += (int64_t)gridDim.x * 256)
        ws[i] = (i == 1 || i == 2) ? 0x7fffffff : 0;
}

__global__ __launch_bounds__(256) void token_plan_count_kernel(TokenLaunch a, int32_t *ws) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n) return;
    const int r0 = a.src0[i], r1 = a.src1[i];
    bool bad = false;
    if ((uint32_t)r0 < (uint32_t)a.L)
        atomicAdd(&ws[3 + r0], 1);
    else
        bad = true;
    if ((uint32_t)r1 < (uint32_t)a.L)
        atomicAdd(&ws[3 + r1], 1);
    else if (r1 != -1)
        bad = true;
    if (bad) {
        atomicOr(&ws[0], PMA_PLAN_BAD_INDEX);
        atomicMin(&ws[1], i);
    }
}

__global__ __launch_bounds__(256) void token_plan_rows_kernel(int32_t *ws, int32_t L) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= L) return;
    const int c = ws[3 + r];
    if (c == 1) return;
    atomicOr(&ws[0], c == 0 ? PMA_PLAN_ROW_MISSING : PMA_PLAN_ROW_REPEATED);
    atomicMin(&ws[2], r);
}

}  // namespace

hipError_t launch_token_plan_check(const TokenLaunch &a, int32_t *ws, hipStream_t s) {
    const int64_t words = (int64_t)a.L + 3;
    token_plan_clear_kernel<<<(unsigned)std::min<int64_t>((words + 255) / 256, 1024), 256, 0, s>>>(ws, a.L);
    if (a.n > 0) token_plan_count_kernel<<<(a.n + 255) / 256, 256, 0, s>>>(a, ws);
    token_plan_rows_kernel<<<(a.L + 255) / 256, 256, 0, s>>>(ws, a.L);
    return hipGetLastError();
}

hipError_t launch_token_merge(const TokenLaunch &a, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    token_merge_kernel<<<a.n, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_token_restore(const TokenLaunch &a, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    token_restore_kernel<<<a.n, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace pma
