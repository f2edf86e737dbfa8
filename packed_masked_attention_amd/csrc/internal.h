// internal.h -- types and launchers shared by the libpma translation units.
// gfx950 only: wave64, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pma.h"

namespace pma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;   // the only head size the kernels are built for
constexpr int kPadRows = 256;   // attention operands are padded to a multiple of this

// bf16 bits <-> fp32 (exact widening; RNE narrowing through the hardware convert)
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// ------------------------------------------------------------------ layout
struct LayoutLaunch {
    int32_t L, T, tile_m, tile_n, nqt, nkt;
    const int32_t *tags, *pos, *ts_idx;
    const int32_t *vid, *aud, *txt;
    int32_t nv, na, nt;
    int32_t *doc;
    uint8_t *cls;
    int32_t *count, *list, *order, *status;
    int32_t *scratch;  // [0..2] tag counts, then q-tile flags [nqt], k-tile flags [nkt]
};
hipError_t launch_layout_build(const LayoutLaunch &a, hipStream_t s);

// ------------------------------------------------------------- norm + rope
struct PrepLaunch {
    int32_t L, Lp, H, F;
    float eps;
    float qscale;           // factor on Q' (the attention operand's logit scale)
    double inv_freq[16];
    double pos_scale[3];    // per-axis scale of the positions (1 = integer positions)
    const uint16_t *q, *k, *v;
    int64_t q_ld, k_ld, v_ld;
    const float *wq, *wk;
    const int32_t *pos;
    uint16_t *qh, *kh, *vt;
};
hipError_t launch_qk_norm_rope(const PrepLaunch &a, hipStream_t s);
// (cos, sin) of every row's 3F rotation angles, built in fp64: rope[i][a*F+f]
hipError_t launch_rope_table(const PrepLaunch &a, float2 *rope, hipStream_t s);

// ----------------------------------------------------------------- flash
struct FlashLaunch {
    int32_t L, Lp, H, nqt, nkt;
    const uint16_t *qh, *kh, *vt;   // Q' carries the logit scale softmax_scale * log2(e)
    uint16_t *o;
    int64_t o_ld;
    float *lse;
    const int32_t *doc;
    const uint8_t *cls;
    const int32_t *count, *list, *order;
    // work queue (NULL: one item per workgroup, nothing split): counters of
    // the persistent workgroups, the key-range split of the last split_items
    // items of every XCD's share and their partial results (part)
    int32_t *queue;
    int32_t split_items;   // S: the last S items of every XCD's share run in parts
    float *part;
    // clock stamps of the persistent workgroups (NULL: none): per workgroup
    // {shader clock, 100 MHz real-time clock} at its start and its end
    uint64_t *stamps;
};
// the flash workspace's clock-stamp area: 4 x u64 per persistent workgroup
constexpr int kFlashStampGroups = 1024;
constexpr size_t kFlashStampBytes = (size_t)kFlashStampGroups * 4 * sizeof(uint64_t);
void flash_tiles(int32_t *tile_m, int32_t *tile_n);
// bytes of work-queue counters at the start of the flash workspace
constexpr size_t kFlashQueueBytes = 256;
// items per XCD whose key range is split, and the work-queue bytes (counters
// and partial results) the split needs
int32_t flash_split_items(int32_t H, int32_t L);
size_t flash_split_bytes(int32_t H, int32_t L);
// work-queue counters + partial results of split_items split items per XCD
size_t flash_split_bytes_for(int32_t split_items);
// most k-tiles a layout may have for the attention kernel (its LDS tile list)
int32_t flash_max_k_tiles();
hipError_t launch_flash_attention(const FlashLaunch &a, hipStream_t s);

// ------------------------------------------------------------------ block
struct GemmLaunch {
    int32_t M, N, K;
    const uint16_t *A;
    int64_t lda;
    const uint16_t *W;
    int64_t ldw;
    uint32_t w_bytes;  // bytes of W addressable by the kernel's buffer resource
    uint16_t *C;
    int64_t ldc;
    int32_t epi;
    const uint16_t *R;
    int64_t ldr;
    const float *table;
    int32_t T, gate_chunk;
    const int32_t *tags, *ts_idx;
    // QKV projection epilogue (kEpiQkvRope): per-head RMSNorm + RoPE of the Q
    // and K columns from the fp32 accumulators, head-major Q', K' and V^T out
    int32_t Lp, H, F;
    float eps;
    float qscale;               // factor on Q' (the attention operand's logit scale)
    const float *wq, *wk;       // norm weights [128]
    const float2 *rope;         // (cos, sin) [L][3F]
    uint16_t *qh, *kh, *vt;     // [H][Lp][128], [H][Lp][128], [H][128][Lp]
    // output columns [n_begin, n_end) of this launch (n_end 0: all N);
    // launch_gemm sets them when it splits a problem between tile shapes
    int32_t n_begin, n_end;
    // gated residual with row statistics (kEpiGateStats): per row and column
    // group of gemm_stats_group_width columns, (mean, sum of squared
    // deviations) of the bf16-rounded output row, [M][stats_groups]
    float2 *stats;
    int32_t stats_groups;
};
// internal epilogue ids (beside PMA_EPI_*): the fused QKV projection (3, 4:
// one per rope_freq_dim), and the gated residual that also takes the
// LayerNorm statistics of its rounded output rows
constexpr int kEpiQkvRope = 3;
constexpr int kEpiGateStats = 5;
// Columns per row-statistics group of the kEpiGateStats epilogue (the
// columns one wave of an output tile holds for a row): 224 or 128.
int gemm_stats_group_width(int M, int N);
hipError_t launch_gemm(const GemmLaunch &a, hipStream_t s);
// W rows per output tile launch_gemm takes for this problem (256, or 224
// where that fills the last round of tiles better)
int gemm_tile_n(int epi, int M, int N);
// output columns the fused QKV projection runs as 128-wide tiles in a second
// launch (0: none)
int gemm_qkv_narrow_columns(int M, int N);

struct LnModLaunch {
    int32_t L, hidden, T, shift_chunk;
    float eps;
    const uint16_t *x;
    uint16_t *out;
    const float *table;
    const int32_t *tags, *ts_idx;
    // with stats: the rows' statistics from the kEpiGateStats epilogue
    // (stats_groups groups of stats_gw columns per row) replace the row
    // reductions
    const float2 *stats;
    int32_t stats_groups, stats_gw;
};
hipError_t launch_ln_modulate(const LnModLaunch &a, hipStream_t s);
int ln_modulate_max_hidden();

struct AdaLnLaunch {
    int32_t T, E, hidden;
    const uint16_t *temb, *w;
    float *table;
};
hipError_t launch_adaln_table(const AdaLnLaunch &a, hipStream_t s);
int adaln_max_t();

// ------------------------------------------------------- input / output path
struct GemvLaunch {
    int32_t T, K, N;
    int32_t group_rows;        // out[(g*T + t)*group_rows + n % group_rows], g = n / group_rows
    const float *x;            // [T][K] (unused when timestep is set)
    const float *timestep;     // [T]: x = sinusoid of these (K = freq_dim)
    double log_max_period;
    const float *W;            // [N][K]
    const float *b;            // [N] or null
    int32_t silu;
    float *out;
    uint16_t *out_bf16;        // optional bf16 copy, same layout
};
hipError_t launch_gemv(const GemvLaunch &a, hipStream_t s);
int gemv_max_t();

struct ProjLaunch {
    int32_t rows, K, N, L;     // N % 128 == 0, K % 32 == 0
    const float *X;            // [rows][K]
    const float *W;            // [N][K]
    const float *b;            // [N]
    const int32_t *idx;        // [rows] destination rows
    uint16_t *out;
    int64_t ld_out;
};
hipError_t launch_proj_scatter(const ProjLaunch &a, hipStream_t s);

struct TextScatterLaunch {
    int32_t rows, hidden, L;
    const uint16_t *src;
    int64_t ld_src;
    const int32_t *idx;
    uint16_t *out;
    int64_t ld_out;
};
hipError_t launch_text_scatter(const TextScatterLaunch &a, hipStream_t s);

struct HeadLaunch {
    int32_t rows, hidden, nout, L, T, head, splits;
    float eps;
    const uint16_t *x;
    int64_t ld_x;
    const int32_t *idx, *ts_idx;
    const float *table;        // [2][T][2][hidden]
    const float *W, *b;        // [nout][hidden], [nout]
    float2 *stats;             // [rows]
    float *partial;            // [splits][rows][nout]
    float *out;                // [rows][nout]
};
hipError_t launch_head(const HeadLaunch &a, hipStream_t s);
int head_max_hidden();

// token reduction: merge rows (src0[i], src1[i]) of x into row i of xr_out;
// restore x_out[r] = x[r] + (xr_in[i] - xr_before[i]) for r in {src0, src1}
struct TokenLaunch {
    int32_t n, hidden, L;
    const int32_t *src0, *src1;
    const uint16_t *x;          // full rows (merge input / restore bypass)
    uint16_t *xr_out;           // merge output
    const uint16_t *xr_before, *xr_in;
    uint16_t *x_out;            // restore output (may alias x)
};
hipError_t launch_token_merge(const TokenLaunch &a, hipStream_t s);
// ws: int32 [3 + L] (status bits, first bad entry, first bad row, row counts)
hipError_t launch_token_plan_check(const TokenLaunch &a, int32_t *ws, hipStream_t s);
hipError_t launch_token_restore(const TokenLaunch &a, hipStream_t s);
int head_max_out();
int head_max_t();     // distinct timesteps the head kernels accept
int head_k_chunk();   // each head K range is a multiple of this

}  // namespace pma
