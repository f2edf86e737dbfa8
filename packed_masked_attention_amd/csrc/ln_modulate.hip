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
// HBM-bound: one wave per row reads the row once (kept in registers for both
// passes of the mean/variance), gathers the two fp32 modulation rows (3 x T
// distinct rows, L2-resident) and writes the row once.  After a gated
// residual that took the row statistics in its epilogue (page "MiniMax H3
// Inference Engine voor Mac computers", "Exacte DiT fusions": the residual
// gate fused with the next AdaLN), the mean and variance come from those
// per-group (mean, sum of squared deviations) pairs instead, combined with
// the pairwise update of Chan, Golub and LeVeque (equal group sizes n_g):
// mean = sum mean_g / G, M2 = sum (M2_g + n_g (mean_g - mean)^2).
#include "internal.h"

namespace pma {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;   // one wave per row
constexpr int kMaxChunks = 16;  // 16-byte chunks per lane: hidden <= 64*8*16 = 8192

__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// One wave per row, CPL 16-byte chunks per lane (hidden <= 512 CPL): the row
// stays in registers as bf16 for both passes of the mean/variance, and the
// reductions stay inside the wave (no block barriers; 46 -> 43 us at
// 8192 x 5376 against one 256-thread block per row).
template <int CPL, bool STATS>
__global__ __launch_bounds__(kThreads) void ln_modulate_kernel(LnModLaunch a) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= a.L) return;
    const int nchunk = a.hidden / 8;
    const uint16_t *xr = a.x + (int64_t)row * a.hidden;
    u16x8 raw[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        raw[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (c < nchunk) raw[i] = *reinterpret_cast<const u16x8 *>(xr + 8 * c);
    }
    float mean, var;
    if constexpr (STATS) {
        // lane g < G holds group g's pair (G <= 64: hidden <= 8192, groups of
        // at least 128 columns)
        float2 st = make_float2(0.f, 0.f);
        if (lane < a.stats_groups) st = a.stats[(int64_t)row * a.stats_groups + lane];
        mean = wave_sum(st.x) / (float)a.stats_groups;
        const float d = st.x - mean;
        const float m2 = lane < a.stats_groups ? fmaf((float)a.stats_gw * d, d, st.y) : 0.f;
        var = wave_sum(m2) / (float)a.hidden;
    } else {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int t = 0; t < 8; ++t) s += bf16_bits_to_f32(raw[i][t]);
        mean = wave_sum(s) / (float)a.hidden;
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            if (lane + 64 * i < nchunk) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float d = bf16_bits_to_f32(raw[i][t]) - mean;
                    q = fmaf(d, d, q);
                }
            }
        }
        var = wave_sum(q) / (float)a.hidden;
    }
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
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) {
            float y[8];
            if (shift) {
                const f32x4 sh0 = *reinterpret_cast<const f32x4 *>(shift + 8 * c);
                const f32x4 sh1 = *reinterpret_cast<const f32x4 *>(shift + 8 * c + 4);
                const f32x4 sc0 = *reinterpret_cast<const f32x4 *>(scale + 8 * c);
                const f32x4 sc1 = *reinterpret_cast<const f32x4 *>(scale + 8 * c + 4);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    y[t] = fmaf((bf16_bits_to_f32(raw[i][t]) - mean) * rstd, 1.0f + sc0[t], sh0[t]);
                    y[t + 4] = fmaf((bf16_bits_to_f32(raw[i][t + 4]) - mean) * rstd, 1.0f + sc1[t], sh1[t]);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) y[t] = (bf16_bits_to_f32(raw[i][t]) - mean) * rstd;
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
    const dim3 grid((a.L + kRowsPerBlock - 1) / kRowsPerBlock);
    const int cpl = (a.hidden / 8 + 63) / 64;
    if (a.stats && (a.stats_groups < 1 || a.stats_groups > 64 || a.stats_groups * a.stats_gw != a.hidden))
        return hipErrorInvalidValue;
    if (a.stats) {
        if (cpl <= 4) ln_modulate_kernel<4, true><<<grid, kThreads, 0, s>>>(a);
        else if (cpl <= 8) ln_modulate_kernel<8, true><<<grid, kThreads, 0, s>>>(a);
        else if (cpl <= 12) ln_modulate_kernel<12, true><<<grid, kThreads, 0, s>>>(a);
        else ln_modulate_kernel<16, true><<<grid, kThreads, 0, s>>>(a);
    } else {
        if (cpl <= 4) ln_modulate_kernel<4, false><<<grid, kThreads, 0, s>>>(a);
        else if (cpl <= 8) ln_modulate_kernel<8, false><<<grid, kThreads, 0, s>>>(a);
        else if (cpl <= 12) ln_modulate_kernel<12, false><<<grid, kThreads, 0, s>>>(a);
        else ln_modulate_kernel<16, false><<<grid, kThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

int ln_modulate_max_hidden() { return 64 * 8 * kMaxChunks; }

}  // namespace pma
