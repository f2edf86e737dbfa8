// inout.hip -- the steps either side of the block stack: the timestep MLP, the
// input projections scattered into the packed stream, and the output heads
// gathered from it.
//
// Page "MiniMaxH3Transformer3DModel" (diffusers API page): constructor
// parameters freq_dim (a sinusoidal embedding of the unscaled timestep),
// time_embed_hidden_dim / time_embed_dim (the timestep MLP's inner and output
// widths), in_channels x prod(patch_size) and audio_in_channels (latent row
// widths), final_norm_eps (norm_out); forward parameters (the latent rows are
// ordered as video_indices / audio_indices / text_indices, timestep_indices
// points every row into the distinct timesteps) and returns (velocities in
// the row order of their index tensors); intro (patch projections, timestep
// MLP and output heads are fp32).  Page "MiniMax H3 Inference Engine voor Mac
// computers", implementation notes: the fp32 patch projections round straight
// to bf16 into the packed hidden stream; the final AdaLN reads its rows at
// their offsets in the residual stream and the heads modulate while loading
// their projection tiles.
//
// Readings: embedding = [cos(t w_j) | sin(t w_j)], w_j = max_period^(-j/half);
// MLP = Linear -> SiLU -> Linear with biases; projections and heads are
// Linear with bias; the head applies LN (no affine, eps = final_norm_eps),
// then u * (1 + scale) + shift with (shift, scale) chosen by the row's
// timestep from a per-head table temb @ W_mod^T (no bias).
//
// Kernels:
//  * gemv_kernel -- out[t] = act(W x[t] + b) for T <= 8 vectors of fp32: the
//    MLP layers and the head table.  Bound by reading the fp32 weights once:
//    one wave per weight row streams it with 8 16-byte loads in flight per
//    lane; the T inputs are read through the caches (the first MLP layer
//    builds its sinusoid in LDS, in fp64).
//  * proj_scatter_kernel -- X W^T + b on fp32 MFMA (32x32x2), 128 x 128 tile
//    per 4-wave block, K staged through LDS in chunks of 32; the epilogue
//    rounds to bf16 and writes row i to packed row idx[i].  With K = 96 every
//    output element costs 96 multiply-adds against 2 stored bytes, so the
//    kernel is bound by the fp32 matrix rate, not by HBM.
//  * text_scatter_kernel -- copies the projected text rows to their rows.
//  * head_stats_kernel -- mean and 1/std of every gathered row (one wave each).
//  * head_gemm_kernel -- split-K fp32 MFMA: a wave owns 32 gathered rows and
//    one K range; it loads its operands straight from global memory (16 bytes
//    of x per lane and step), normalises and modulates them in registers and
//    contracts them against every output column; partial sums go to the
//    workspace.
//  * head_finalize_kernel -- sums the K-range partials and adds the bias.
#include "internal.h"

namespace pma {
namespace {

// ------------------------------------------------------------------ GEMV
constexpr int kGemvThreads = 256;   // 4 waves, one weight row each
constexpr int kGemvMaxT = 8;
constexpr int kGemvUnroll = 8;      // 16-byte weight loads in flight per lane

// out[t][n] for one row n per wave: lane l reads W[n][256 i + 4 l .. +4] and
// x[t][...] at the same columns (x is small and cache-resident; the first MLP
// layer reads its sinusoid from LDS instead), then a wave reduction.
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvLaunch a) {
    extern __shared__ __align__(16) float es[];   // [T][K] sinusoid (timestep mode only)
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * (kGemvThreads / 64) + (threadIdx.x >> 6);
    const float *xb = a.x;
    if (a.timestep) {
        // sinusoid of the unscaled timestep, built in fp64: [cos | sin]
        const int half = a.K / 2;
        for (int i = threadIdx.x; i < a.T * a.K; i += kGemvThreads) {
            const int t = i / a.K, k = i - t * a.K;
            const int j = k < half ? k : k - half;
            const double ang = (double)a.timestep[t] * exp(-a.log_max_period * (double)j / half);
            es[i] = (float)(k < half ? cos(ang) : sin(ang));
        }
        __syncthreads();
        xb = es;
    }
    if (n >= a.N) return;
    const float *w = a.W + (int64_t)n * a.K;
    float acc[kGemvMaxT];
#pragma unroll
    for (int t = 0; t < kGemvMaxT; ++t) acc[t] = 0.f;
    int k = 4 * lane;
    for (; k + 256 * (kGemvUnroll - 1) < a.K; k += 256 * kGemvUnroll) {
        f32x4 wv[kGemvUnroll];
#pragma unroll
        for (int u = 0; u < kGemvUnroll; ++u)
            wv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(w + k + 256 * u));
#pragma unroll
        for (int t = 0; t < kGemvMaxT; ++t) {
            if (t < a.T) {
#pragma unroll
                for (int u = 0; u < kGemvUnroll; ++u) {
                    const f32x4 xv = *reinterpret_cast<const f32x4 *>(xb + (int64_t)t * a.K + k + 256 * u);
                    acc[t] = fmaf(wv[u][0], xv[0], acc[t]);
                    acc[t] = fmaf(wv[u][1], xv[1], acc[t]);
                    acc[t] = fmaf(wv[u][2], xv[2], acc[t]);
                    acc[t] = fmaf(wv[u][3], xv[3], acc[t]);
                }
            }
        }
    }
    for (; k < a.K; k += 256) {
        const f32x4 wv = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(w + k));
#pragma unroll
        for (int t = 0; t < kGemvMaxT; ++t) {
            if (t < a.T) {
                const f32x4 xv = *reinterpret_cast<const f32x4 *>(xb + (int64_t)t * a.K + k);
                acc[t] = fmaf(wv[0], xv[0], acc[t]);
                acc[t] = fmaf(wv[1], xv[1], acc[t]);
                acc[t] = fmaf(wv[2], xv[2], acc[t]);
                acc[t] = fmaf(wv[3], xv[3], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kGemvMaxT; ++t) {
        float v = acc[t];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
        acc[t] = v;
    }
    if (lane >= a.T) return;
    float v = acc[0];
#pragma unroll
    for (int t = 1; t < kGemvMaxT; ++t) if (lane == t) v = acc[t];
    if (a.b) v += a.b[n];
    if (a.silu) v = v / (1.0f + expf(-v));
    // row n of group g = n / group_rows lands at out[(g * T + t) * group_rows + n % group_rows]
    const int g = n / a.group_rows, r = n - g * a.group_rows;
    const int64_t o = ((int64_t)g * a.T + lane) * a.group_rows + r;
    a.out[o] = v;
    if (a.out_bf16) {
        f32x2 p = {v, 0.f};
        a.out_bf16[o] = __builtin_bit_cast(uint16_t, __builtin_convertvector(p, bf16x2)[0]);
    }
}

// ------------------------------------------------- projection + scatter
constexpr int kProjThreads = 256;
constexpr int kProjRows = 128;     // data rows per block (2 waves x 2 tiles of 32)
constexpr int kProjCols = 128;     // output columns per block (2 waves x 2 tiles of 32)
constexpr int kProjKc = 32;        // K per LDS chunk
constexpr int kProjPitch = kProjKc + 1;
constexpr int kProjOutPitch = kProjCols + 8;   // bf16 per staged output row (16-byte rows, 2-way banks)
// operand tiles during the K loop, the bf16 output tile after it
constexpr int kProjSmemFloats =
    (2 * kProjRows * kProjPitch > kProjRows * kProjOutPitch / 2) ? 2 * kProjRows * kProjPitch
                                                                 : kProjRows * kProjOutPitch / 2;

// Wider tiles (128 x 256 per block) measured slower: fewer resident waves.
__global__ __launch_bounds__(kProjThreads) __attribute__((amdgpu_waves_per_eu(2)))
void proj_scatter_kernel(ProjLaunch a) {
    constexpr int NTW = 2;             // column tiles of 32 per wave
    constexpr int kCols = kProjCols;
    __shared__ __align__(16) float smem[kProjSmemFloats];
    __shared__ int32_t dst[kProjRows];
    float *as = smem, *bs = smem + kProjRows * kProjPitch;
    static_assert(kCols == kProjRows, "the two operand tiles share one buffer");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // XCD-aware order: the dispatcher deals workgroups round-robin to the 8
    // XCDs, so workgroup b takes item (b % 8) * per_xcd + b / 8; items run
    // row tiles fastest, so an XCD sweeps a few column tiles (weights) over
    // every row tile (inputs), both L2-resident
    const int row_tiles = (a.rows + kProjRows - 1) / kProjRows;
    const int total = row_tiles * (a.N / kCols);
    const int per_xcd = (total + 7) / 8;
    const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (item >= total) return;
    const int r0 = (item % row_tiles) * kProjRows, n0 = (item / row_tiles) * kCols;
    if (tid < kProjRows) {
        const int r = r0 + tid;
        int d = -1;
        if (r < a.rows) {
            d = a.idx[r];
            if ((uint32_t)d >= (uint32_t)a.L) d = -1;   // out-of-range entries are skipped
        }
        dst[tid] = d;
    }
    f32x16 acc[2][NTW];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    const int kq = tid & 7, rr = tid >> 3;   // float4 column within the chunk, row within 32
    const int l32 = lane & 31, hk = lane >> 5;
    // the next chunk's global loads are issued before this chunk's MFMAs
    f32x4 xv[kProjRows / 32], wv[kCols / 32];
    auto load = [&](int k0) {
#pragma unroll
        for (int j = 0; j < kProjRows / 32; ++j) {
            const int row = rr + 32 * j;
            xv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (r0 + row < a.rows)
                xv[j] = *reinterpret_cast<const f32x4 *>(a.X + (int64_t)(r0 + row) * a.K + k0 + 4 * kq);
        }
#pragma unroll
        for (int j = 0; j < kCols / 32; ++j)
            wv[j] = *reinterpret_cast<const f32x4 *>(a.W + (int64_t)(n0 + rr + 32 * j) * a.K + k0 + 4 * kq);
    };
    load(0);
    for (int k0 = 0; k0 < a.K; k0 += kProjKc) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kProjRows / 32; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) as[(rr + 32 * j) * kProjPitch + 4 * kq + e] = xv[j][e];
#pragma unroll
        for (int j = 0; j < kCols / 32; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) bs[(rr + 32 * j) * kProjPitch + 4 * kq + e] = wv[j][e];
        __syncthreads();
        if (k0 + kProjKc < a.K) load(k0 + kProjKc);
#pragma unroll 4
        for (int kk = 0; kk < kProjKc; kk += 2) {
            float av[2], bv[NTW];
#pragma unroll
            for (int i = 0; i < 2; ++i) av[i] = as[(64 * wm + 32 * i + l32) * kProjPitch + kk + hk];
#pragma unroll
            for (int j = 0; j < NTW; ++j)
                bv[j] = bs[(32 * NTW * wn + 32 * j + l32) * kProjPitch + kk + hk];
            // transposed product: the weight rows are the MFMA's rows, the data
            // rows its columns, so a lane ends up holding one data row
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NTW; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[j], av[i], acc[i][j], 0, 0, 0);
        }
    }
    // D register v of tile (i, j): output column 8(v/4) + 4(lane/32) + v%4 of
    // column tile j, data row lane%32 of row tile i -> 4 adjacent columns per
    // group of 4 registers.  The bf16 tile goes through LDS so that every
    // global store covers whole 128-byte lines (a partial line would make the
    // L2 fetch the rest of it).
    __syncthreads();   // every wave is done with the operand tiles
    uint16_t *ot = reinterpret_cast<uint16_t *>(smem);   // [128 rows][kProjOutPitch]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 64 * wm + 32 * i + l32;
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = 32 * NTW * wn + 32 * j + 8 * g + 4 * hk;
                const f32x4 bias = *reinterpret_cast<const f32x4 *>(a.b + n0 + c);
                uint2 w;
                w.x = pack_bf16x2(acc[i][j][4 * g] + bias[0], acc[i][j][4 * g + 1] + bias[1]);
                w.y = pack_bf16x2(acc[i][j][4 * g + 2] + bias[2], acc[i][j][4 * g + 3] + bias[3]);
                *reinterpret_cast<uint2 *>(ot + row * kProjOutPitch + c) = w;
            }
        }
    }
    __syncthreads();
    // 16 threads per 256-byte row segment, 16 rows per pass
#pragma unroll
    for (int it = 0; it < kProjRows / 16; ++it) {
        const int row = it * 16 + (tid >> 4), ch = tid & 15;
        const int d = dst[row];
        if (d >= 0)
            *reinterpret_cast<uint4 *>(a.out + (int64_t)d * a.ld_out + n0 + 8 * ch) =
                *reinterpret_cast<const uint4 *>(ot + row * kProjOutPitch + 8 * ch);
    }
}

// ------------------------------------------------------------ text scatter
__global__ __launch_bounds__(256) void text_scatter_kernel(TextScatterLaunch a) {
    const int i = blockIdx.x;
    const int d = a.idx[i];
    if ((uint32_t)d >= (uint32_t)a.L) return;
    const uint16_t *src = a.src + (int64_t)i * a.ld_src;
    uint16_t *out = a.out + (int64_t)d * a.ld_out;
    for (int c = 8 * threadIdx.x; c < a.hidden; c += 8 * 256)
        *reinterpret_cast<u16x8 *>(out + c) = *reinterpret_cast<const u16x8 *>(src + c);
}

// ------------------------------------------------------------- head stats
constexpr int kStatsMaxChunks = 16;   // 16-byte chunks per lane: hidden <= 64*8*16 = 8192

__global__ __launch_bounds__(256) void head_stats_kernel(HeadLaunch a) {
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= a.rows) return;
    int d = a.idx[i];
    const bool ok = (uint32_t)d < (uint32_t)a.L;
    if (!ok) d = 0;
    const uint16_t *xr = a.x + (int64_t)d * a.ld_x;
    const int nchunk = a.hidden / 8;
    u16x8 raw[kStatsMaxChunks];   // the row stays in registers as bf16 for both passes
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kStatsMaxChunks; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk) {
            raw[c] = *reinterpret_cast<const u16x8 *>(xr + 8 * ch);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += bf16_bits_to_f32(raw[c][e]);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    const float mean = s / (float)a.hidden;
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < kStatsMaxChunks; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dv = bf16_bits_to_f32(raw[c][e]) - mean;
                q = fmaf(dv, dv, q);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) q += __shfl_xor(q, off);
    if (lane == 0) {
        const float rstd = 1.0f / sqrtf(q / (float)a.hidden + a.eps);
        // rows whose index is out of range produce zeros (mean 0, rstd 0)
        a.stats[i] = ok ? make_float2(mean, rstd) : make_float2(0.f, 0.f);
    }
}

// -------------------------------------------------------------- head GEMM
constexpr int kHeadMaxNt = 4;   // output columns <= 128
constexpr int kHeadKc = 64;     // K columns staged in LDS per chunk
constexpr int kHeadPitch = kHeadKc + 4;   // floats per LDS row: 16-byte reads stay conflict-free
constexpr int kHeadMaxT = 8;

// Block = 4 waves = 128 gathered rows, one K range; the weight rows of the
// chunk and the (shift, scale) rows of every timestep sit in LDS, shared by
// the 4 waves; each lane streams 16 bytes of its row per step.
template <int NT>
__global__ __launch_bounds__(256) void head_gemm_kernel(HeadLaunch a) {
    __shared__ __align__(16) float wls[NT * 32 * kHeadPitch];
    __shared__ __align__(16) float tls[kHeadMaxT * 2 * kHeadPitch];
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hk = lane >> 5;
    const int tile = blockIdx.x * 4 + (tid >> 6);
    const int s = blockIdx.y;
    const int i = tile * 32 + l32;
    const bool live = i < a.rows;
    int d = live ? a.idx[i] : 0;
    const bool ok = live && (uint32_t)d < (uint32_t)a.L;   // otherwise the row is zero
    if (!ok) d = 0;
    const float2 st = ok ? a.stats[i] : make_float2(0.f, 0.f);
    const int ts = ok ? a.ts_idx[d] : -1;
    const bool mod = (uint32_t)ts < (uint32_t)a.T;
    const float *tab = a.table + (int64_t)a.head * a.T * 2 * a.hidden;   // [T][2][hidden]
    const float *tl = tls + (mod ? ts : 0) * 2 * kHeadPitch;
    const uint16_t *xr = a.x + (int64_t)d * a.ld_x;
    const int kr = a.hidden / a.splits;
    const int kbeg = s * kr;
    const bool any = tile * 32 < a.rows;    // waves past the last row still join the barriers
    f32x16 acc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    u16x8 xn = *reinterpret_cast<const u16x8 *>(xr + kbeg + 8 * hk);
    for (int k0 = kbeg; k0 < kbeg + kr; k0 += kHeadKc) {
        __syncthreads();
        // weight rows [32 NT][64] and table rows [T][2][64] of this chunk
        for (int q = tid; q < NT * 32 * (kHeadKc / 4); q += 256) {
            const int r = q / (kHeadKc / 4), c4 = q % (kHeadKc / 4);
            *reinterpret_cast<f32x4 *>(wls + r * kHeadPitch + 4 * c4) =
                *reinterpret_cast<const f32x4 *>(a.W + (int64_t)r * a.hidden + k0 + 4 * c4);
        }
        for (int q = tid; q < a.T * 2 * (kHeadKc / 4); q += 256) {
            const int r = q / (kHeadKc / 4), c4 = q % (kHeadKc / 4);
            *reinterpret_cast<f32x4 *>(tls + r * kHeadPitch + 4 * c4) =
                *reinterpret_cast<const f32x4 *>(tab + (int64_t)r * a.hidden + k0 + 4 * c4);
        }
        __syncthreads();
        if (any) {
            // step of 16 k: lane half hk holds k = kb + 8*hk + e for e = 0..7, and the
            // MFMA of index e contracts the pair (kb + e, kb + 8 + e) on both operands
#pragma unroll 2
            for (int kk = 0; kk < kHeadKc; kk += 16) {
                const u16x8 raw = xn;
                const int knext = k0 + kk + 16;
                if (knext < kbeg + kr) xn = *reinterpret_cast<const u16x8 *>(xr + knext + 8 * hk);
                const int kl = kk + 8 * hk;
                const f32x4 sh0 = *reinterpret_cast<const f32x4 *>(tl + kl);
                const f32x4 sh1 = *reinterpret_cast<const f32x4 *>(tl + kl + 4);
                const f32x4 sc0 = *reinterpret_cast<const f32x4 *>(tl + kHeadPitch + kl);
                const f32x4 sc1 = *reinterpret_cast<const f32x4 *>(tl + kHeadPitch + kl + 4);
                float av[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float n = (bf16_bits_to_f32(raw[e]) - st.x) * st.y;
                    const float sc = e < 4 ? sc0[e & 3] : sc1[e & 3];
                    const float sh = e < 4 ? sh0[e & 3] : sh1[e & 3];
                    av[e] = ok ? (mod ? fmaf(n, 1.0f + sc, sh) : n) : 0.f;
                }
                f32x4 wv[NT][2];
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    const float *w = wls + (32 * c + l32) * kHeadPitch + kl;
                    wv[c][0] = *reinterpret_cast<const f32x4 *>(w);
                    wv[c][1] = *reinterpret_cast<const f32x4 *>(w + 4);
                }
                // column tiles innermost: consecutive MFMAs use different accumulators
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int c = 0; c < NT; ++c)
                        acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], wv[c][e >> 2][e & 3],
                                                                      acc[c], 0, 0, 0);
            }
        }
    }
    if (!any) return;
    // partial[s][row][col]; D register v: row 8(v/4) + 4 hk + v%4, column l32
    float *part = a.partial + (int64_t)s * a.rows * a.nout;
#pragma unroll
    for (int c = 0; c < NT; ++c) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = tile * 32 + 8 * (v >> 2) + 4 * hk + (v & 3);
            if (row < a.rows) part[(int64_t)row * a.nout + 32 * c + l32] = acc[c][v];
        }
    }
}

__global__ __launch_bounds__(256) void head_finalize_kernel(HeadLaunch a) {
    const int64_t n = (int64_t)a.rows * a.nout;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    const int col = (int)(e % a.nout);
    // several independent partial sums keep loads in flight
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 8 <= a.splits; s += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] += a.partial[(int64_t)(s + u) * n + e];
    }
    for (; s < a.splits; ++s) v[0] += a.partial[(int64_t)s * n + e];
    a.out[e] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])) + a.b[col];
}

}  // namespace

hipError_t launch_gemv(const GemvLaunch &a, hipStream_t s) {
    const int rows = kGemvThreads / 64;
    const int blocks = (a.N + rows - 1) / rows;
    const size_t lds = a.timestep ? (size_t)a.T * a.K * sizeof(float) : 0;
    gemv_kernel<<<blocks, kGemvThreads, lds, s>>>(a);
    return hipGetLastError();
}

int gemv_max_t() { return kGemvMaxT; }

hipError_t launch_proj_scatter(const ProjLaunch &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    const int total = ((a.rows + kProjRows - 1) / kProjRows) * (a.N / kProjCols);
    proj_scatter_kernel<<<8 * ((total + 7) / 8), kProjThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_text_scatter(const TextScatterLaunch &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    text_scatter_kernel<<<a.rows, 256, 0, s>>>(a);
    return hipGetLastError();
}

int head_max_hidden() { return 64 * 8 * kStatsMaxChunks; }
int head_max_out() { return 32 * kHeadMaxNt; }
int head_max_t() { return kHeadMaxT; }
int head_k_chunk() { return kHeadKc; }

hipError_t launch_head(const HeadLaunch &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    head_stats_kernel<<<(a.rows + 3) / 4, 256, 0, s>>>(a);
    dim3 grid((a.rows + 127) / 128, a.splits);
    switch (a.nout / 32) {
    case 1: head_gemm_kernel<1><<<grid, 256, 0, s>>>(a); break;
    case 2: head_gemm_kernel<2><<<grid, 256, 0, s>>>(a); break;
    case 3: head_gemm_kernel<3><<<grid, 256, 0, s>>>(a); break;
    case 4: head_gemm_kernel<4><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    const int64_t n = (int64_t)a.rows * a.nout;
    head_finalize_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace pma
