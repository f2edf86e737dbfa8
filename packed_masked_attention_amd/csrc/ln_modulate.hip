// ln_modulate.hip -- pre-norm + AdaLN modulation gathered by (tag, timestep).
//
// Page "MiniMaxH3Transformer3DModel" (diffusers API page): intro -- the per-row
// modality tag selects the AdaLN modulation parameters; constructor
// parameters -- norm_eps of the pre-attention and pre-feed-forward norms;
// forward parameters -- token_tags and timestep_indices per row.
// Readings: LayerNorm without affine (population variance), then
// u * (1 + scale) + shift with (shift, scale) = table[tag][ts][chunk];
// padding rows (tag -1) use zero modulation; without a table (the token
// refiner's output norm) every row is normalised only.
//
// HBM-bound: one 256-thread block per row reads the row once (kept in
// registers for both passes of the mean/variance), gathers the two fp32
// modulation rows (3 x T distinct rows, L2-resident) and writes the row once.
#include "internal.h"

namespace pma {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 4;   // 16-byte chunks per thread: hidden <= 256*8*4 = 8192

__device__ __forceinline__ float block_sum(float v, float *red) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t += red[w];
    return t;
}

__global__ __launch_bounds__(kThreads) void ln_modulate_kernel(LnModLaunch a) {
    __shared__ float red[kThreads / 64];
    const int row = blockIdx.x;
    const int nchunk = a.hidden / 8;
    const uint16_t *xr = a.x + (int64_t)row * a.hidden;
    float v[kMaxChunks][8];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
        const int c = threadIdx.x + i * kThreads;
        if (c < nchunk) {
            const u16x8 raw = *reinterpret_cast<const u16x8 *>(xr + 8 * c);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                v[i][t] = bf16_bits_to_f32(raw[t]);
                s += v[i][t];
            }
        }
    }
    const float mean = block_sum(s, red) / (float)a.hidden;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
        const int c = threadIdx.x + i * kThreads;
        if (c < nchunk) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float d = v[i][t] - mean;
                q = fmaf(d, d, q);
            }
        }
    }
    const float var = block_sum(q, red) / (float)a.hidden;
    const float rstd = 1.0f / sqrtf(var + a.eps);
    const int tag = a.tags[row], ts = a.ts_idx[row];
    const float *shift = nullptr, *scale = nullptr;
    if (a.table && tag >= 0 && tag <= 2 && (uint32_t)ts < (uint32_t)a.T) {
        const int64_t base = (int64_t)(tag * a.T + ts) * 6;
        shift = a.table + (base + a.shift_chunk) * a.hidden;
        scale = a.table + (base + a.shift_chunk + 1) * a.hidden;
    }
    uint16_t *orow = a.out + (int64_t)row * a.hidden;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
        const int c = threadIdx.x + i * kThreads;
        if (c < nchunk) {
            float y[8];
            if (shift) {
                const f32x4 sh0 = *reinterpret_cast<const f32x4 *>(shift + 8 * c);
                const f32x4 sh1 = *reinterpret_cast<const f32x4 *>(shift + 8 * c + 4);
                const f32x4 sc0 = *reinterpret_cast<const f32x4 *>(scale + 8 * c);
                const f32x4 sc1 = *reinterpret_cast<const f32x4 *>(scale + 8 * c + 4);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    y[t] = fmaf((v[i][t] - mean) * rstd, 1.0f + sc0[t], sh0[t]);
                    y[t + 4] = fmaf((v[i][t + 4] - mean) * rstd, 1.0f + sc1[t], sh1[t]);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) y[t] = (v[i][t] - mean) * rstd;
            }
            uint4 w;
            w.x = pack_bf16x2(y[0], y[1]);
            w.y = pack_bf16x2(y[2], y[3]);
            w.z = pack_bf16x2(y[4], y[5]);
            w.w = pack_bf16x2(y[6], y[7]);
            *reinterpret_cast<uint4 *>(orow + 8 * c) = w;
        }
    }
}

}  // namespace

hipError_t launch_ln_modulate(const LnModLaunch &a, hipStream_t s) {
    ln_modulate_kernel<<<a.L, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

int ln_modulate_max_hidden() { return kThreads * 8 * kMaxChunks; }

}  // namespace pma
