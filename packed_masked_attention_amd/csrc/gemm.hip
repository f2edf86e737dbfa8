// gemm.hip -- bf16 MFMA GEMM C = epilogue(A W^T) for the DiT block projections.
//
// Page "MiniMaxH3Transformer3DModel" (diffusers API page), constructor
// parameters: hidden_size, num_attention_heads x attention_head_dim (the QKV
// and output projections), ffn_dim of the SwiGLU feed-forward; intro: the
// block stack runs in bf16.  Page "MiniMax H3 Inference Engine voor Mac
// computers", implementation notes: fc1 -> SwiGLU -> fc2, and the gated
// residual written as exact bf16.
//
// Epilogues fused into the store:
//   STORE          C = acc                                (plain projection)
//   GATE_RESIDUAL  C = R + gate[tag, ts] * acc            (O-projection, fc2)
//   GATE_STATS     GATE_RESIDUAL, and per row the LayerNorm statistics of
//                  the rounded C row over the columns a wave holds (its mean
//                  and sum of squared deviations, two passes over registers),
//                  so the next norm needs no reduction over the row.
//                  Page "MiniMax H3 Inference Engine voor Mac computers",
//                  "Exacte DiT fusions": the residual gate fused with the
//                  next AdaLN, the rounded row kept on chip for its norm.
//   SWIGLU         C = silu(acc over gate rows) * acc over the matching up rows (fc1)
//   QKV_ROPE       the QKV projection straight into the attention operands: the
//                  Q and K columns are RMS-normalised per (row, head) and
//                  rotated (3-axis RoPE) from the fp32 accumulators, written
//                  head-major (Q' times the attention's logit scale
//                  softmax_scale * log2 e); the V columns are written
//                  transposed (V^T).
//                  Page "MiniMax H3 Inference Engine voor Mac computers",
//                  checkpoint layout notes: the QK normalisation and RoPE run
//                  fused on the projection output.
//
// Design: 256 x 256 output tile (SWIGLU: 256 rows x 128 outputs built from
// 128 gate rows + 128 up rows of W), four waves (one per SIMD) in a 2 x 2
// grid, each owning a 128 x 128 block as 4 x 4 MFMA 32x32x16 tiles: 256 fp32
// accumulators per lane, which live in the accumulation registers, and per
// 16-deep k-step 16 independent MFMAs on 8 fragment reads (0.5 KB of LDS per
// MFMA).  The MFMA computes D = W A^T (weights as the A operand), so a lane's
// accumulator column is one output ROW: per-row epilogue data (tag, timestep,
// residual row) is lane-constant and each lane writes runs of 4 consecutive
// bf16.  Both operand tiles stream into LDS with buffer_load ... lds (rows
// past M read as zero through the buffer bound) in 64-deep K stages (full
// 128-byte rows per DMA lane group), through a ring of five 32 KB slots, one
// operand half-stage each (the whole 160 KB of LDS): one barrier per stage,
// placed before its last k-step, lets that k-step read the next stage's
// first fragments and frees the stage's two slots.  With a fifth slot the
// next halves can be requested from that barrier on, so a stage's 16 DMA
// instructions per wave spread over four k-steps instead of one, and each
// half still has at least two k-steps of MFMAs to land.  The loop is
// unrolled over the ring's period of five stages (a template parameter
// carries the stage count mod 5, so every slot index is a compile-time
// constant, and the remaining stages run unrolled ahead of the loop or
// behind it).  16-byte chunks are XOR-swizzled by row so the fragment reads
// are bank-conflict-free.  Tiles are ordered in groups of 8 row-tiles and
// dealt out XCD-aware so each XCD works on a compact region sharing A and W
// panels in its L2.  Two more tile shapes fill the CUs' last round better
// (see Tile below): 256 x 224 for the store and gated-residual epilogues, and
// 256 x 128 for the last columns of the QKV projection, in a second launch.
// With the store and SwiGLU epilogues on 256-wide tiles one persistent
// workgroup per CU runs its XCD's tiles in turn and requests the next tile's
// first stages before the current tile's epilogue.
#include "internal.h"

#include <atomic>

namespace pma {
namespace {

constexpr int kNW = 4;         // waves per workgroup, one per SIMD
constexpr int kTM = 256;       // rows of A per tile
constexpr int kTK = 64;        // K per stage
constexpr int kStageElems = kTM * kTK;  // 16384 bf16 = 32 KB per operand half-stage (one slot)
constexpr int kGroupM = 8;
static_assert(kTM * kTK * 2 == 32 * 1024, "32 wave-instructions of 1 KB per A half-stage");

// This wave's DMA instructions, all but the newest n, have landed; then the
// workgroup barrier (a plain s_barrier: the release fence of __syncthreads()
// would wait for every DMA in flight)
#define PMA_STAGE_END(n)                                                                    \
    do {                                                                                     \
        __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14)); \
        asm volatile("s_barrier" ::: "memory");                                             \
    } while (0)
constexpr int kRsrcFlags = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void;

// LDS position of 16-byte chunk c (0..7) of tile row r (128-byte rows).  A
// 16-byte fragment read is served 16 lanes (16 consecutive rows, one chunk)
// per cycle from 256 bytes of banks; rotating the chunk by (r >> 1) & 7 puts
// those 16 rows' chunks in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int g_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_void *l, uint32_t voff,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcFlags);
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (1 ulp) instead of an
// IEEE division: the product is rounded to bf16 (2^-9) right after, and the
// division's scale-and-fixup sequence was most of the SwiGLU epilogue's VALU
// work.  e^-z = inf gives z * 0 (the limit), e^-z = 0 gives z.
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// QKV_ROPE epilogue ids: one per rope_freq_dim F (the partner of a rotated
// channel sits F/2 accumulator registers away in the same lane)
constexpr int kEpiQkvF16 = kEpiQkvRope;
constexpr int kEpiQkvF8 = kEpiQkvRope + 1;

// The QKV projection's epilogue.  The tile lies inside one of Q, K, V (H
// even): a 256-column tile holds two heads and wave (wm, wn) has tokens
// m0 + 128 wm + [0, 128) of head wn (FI = 4); a 128-column tile holds one
// head and wave wm has tokens m0 + 64 wm + [0, 64) (FI = 2, wn = 0).  A
// lane's registers for one token: acc[i][j][v] = channel 32 j + 8 (v / 4) +
// 4 hi + v % 4 of token m0 + 32 FI wm + 32 i + l32.  Rows past the sequence
// have all-zero accumulators (their A rows read as zero), so the padding rows
// up to Lp come out as zeros.  st: this wave's LDS (32 FI x 256 bytes) for
// the V^T staging.
template <int F, int FI>
__device__ __forceinline__ void qkv_epilogue(const GemmLaunch &a, f32x16 (&acc)[FI][4], int m0,
                                             int n0, int wm, int wn, int l32, int hi,
                                             uint16_t *st) {
    constexpr int TOK = 32 * FI;                       // tokens of a wave
    const int HD = a.H * kHeadDim;
    const int tensor = n0 / HD;                        // 0 Q, 1 K, 2 V
    const int head = (n0 - tensor * HD) / kHeadDim + wn;
    if (tensor < 2) {
        const float *w = tensor ? a.wk : a.wq;
        uint16_t *dst = (tensor ? a.kh : a.qh) + (int64_t)head * a.Lp * kHeadDim;
        // Q' also carries the attention's logit scale
        const float fac = tensor ? 1.0f : a.qscale;
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            // sum of squares of the token's 128 channels: the lane's 64, then
            // the other lane half's 64
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) t = fmaf(acc[i][j][v], acc[i][j][v], t);
            const uint32_t u = __float_as_uint(t);
            const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            const float tot = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            const float rn = fac / sqrtf(tot * (1.0f / kHeadDim) + a.eps);
            const int m = m0 + TOK * wm + 32 * i + l32;
            // rows past the sequence are zero: any in-range table row serves
            const float2 *rope = a.rope + (int64_t)min(m, a.M - 1) * 3 * F;
            uint16_t *drow = dst + (int64_t)m * kHeadDim + 4 * hi;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float n[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 wv = *reinterpret_cast<const f32x4 *>(w + 32 * j + 8 * g + 4 * hi);
#pragma unroll
                    for (int e = 0; e < 4; ++e) n[4 * g + e] = acc[i][j][4 * g + e] * rn * wv[e];
                }
                float y[16];
                // registers v = 4 q + e hold channel 32 j + 8 q + 4 hi + e; a group
                // of four is wholly rotated (c < 6F, four consecutive angles of
                // one section, partner F/2 registers away) or wholly passed on
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = 32 * j + 8 * q + 4 * hi;
                    if (c < 6 * F) {
                        const int sec = c / (2 * F), f = c % F;
                        const bool first = ((q & (F >> 3)) == 0);
                        const f32x4 lo = *reinterpret_cast<const f32x4 *>(rope + sec * F + f);
                        const f32x4 up = *reinterpret_cast<const f32x4 *>(rope + sec * F + f + 2);
                        const float co[4] = {lo[0], lo[2], up[0], up[2]};
                        const float si[4] = {lo[1], lo[3], up[1], up[3]};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int v = 4 * q + e;
                            const float pn = n[v ^ (F / 2)];
                            y[v] = first ? n[v] * co[e] - pn * si[e] : n[v] * co[e] + pn * si[e];
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[4 * q + e] = n[4 * q + e];
                    }
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint2 o;
                    o.x = pack_bf16x2(y[4 * g], y[4 * g + 1]);
                    o.y = pack_bf16x2(y[4 * g + 2], y[4 * g + 3]);
                    *reinterpret_cast<uint2 *>(drow + 32 * j + 8 * g) = o;
                }
            }
        }
    } else {
        // V^T: each wave stages its 128 channels x TOK tokens in its own LDS
        // (st), then writes channel rows of TOK tokens (2 TOK contiguous bytes)
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int cl = 32 * j + 8 * (v / 4) + 4 * hi + v % 4;
                    st[cl * TOK + 32 * i + l32] = (uint16_t)(pack_bf16x2(acc[i][j][v], 0.f) & 0xffffu);
                }
        // the wave reads back only what it wrote; LDS keeps a wave's accesses in order
        const int lane = l32 + 32 * hi;
        constexpr int CPR = TOK / 8;                   // 16-byte chunks per channel row
        uint16_t *vbase = a.vt + (int64_t)head * kHeadDim * a.Lp + m0 + TOK * wm;
#pragma unroll
        for (int it = 0; it < kHeadDim * CPR / 64; ++it) {
            const int row = it * (64 / CPR) + lane / CPR, ch = lane % CPR;
            const uint4 val = *reinterpret_cast<const uint4 *>(st + row * TOK + ch * 8);
            *reinterpret_cast<uint4 *>(vbase + (int64_t)row * a.Lp + ch * 8) = val;
        }
    }
}

// Tile shapes: 256 rows of A times TN rows of W.  TN = 256: four waves in a
// 2 x 2 grid, 4 x 4 MFMA tiles each; TN = 224 (only the STORE and
// GATE_RESIDUAL epilogues): four waves stacked along M, 2 x 7 MFMA tiles each
// (64 rows x all 224 W rows), for N where 224-wide tiles fill the CUs'
// last round of tiles better (N = 5376: 768 tiles, three full rounds on 256
// CUs, against 672 = 2.625 rounds of 256-wide tiles).
// Sum of a value over the lane pair (l, l ^ 32): v_permlane32_swap leaves
// {own, partner} in the two results.
__device__ __forceinline__ float pair_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int TN> struct Tile;
template <> struct Tile<256> { static constexpr int WM = 2, FI = 4, FJ = 4; };
template <> struct Tile<224> { static constexpr int WM = 4, FI = 2, FJ = 7; };
// 256 x 128 (the QKV epilogue only): four waves stacked along M, 2 x 4 MFMA
// tiles each (64 tokens x one head), for the columns of a partial last round
template <> struct Tile<128> { static constexpr int WM = 4, FI = 2, FJ = 4; };

// The DMA schedule of the interval between the barriers of stages s-1 and s:
// per wave the W half of stage s+1 (TN/32 instructions, first) and the A half
// of stage s+2 (8), four in k-step 3 of stage s-1 and the rest spread over
// k-steps 0..2 of stage s, each k-step's share evenly over its MFMAs (rather
// than a stage's 16 in one k-step: that fills the vector memory path and the
// MFMA issue stalls behind it).
template <int TN> struct Sched {
    static constexpr int NW = TN / 32;            // W instructions per wave per half
    static constexpr int NQ = NW + 8;             // interval positions
    // k-step 3 (previous stage), then k-steps 0, 1, 2 (4,4,4,4 / 4,4,4,3 / 4,3,3,2)
    static constexpr int n[4] = {4, (NQ - 2) / 3, (NQ - 3) / 3, (NQ - 4) / 3};
    static constexpr int first(int q) { return q == 0 ? 0 : first(q - 1) + n[q - 1]; }
    static_assert(n[0] + n[1] + n[2] + n[3] == NQ && n[3] >= 1 && n[0] <= NW,
                  "every position once, the W half leading the interval");
};

template <int EPI, int R, int TN>
__global__ __launch_bounds__(kNW * 64, 1) void gemm_kernel(GemmLaunch a) {
    using T = Tile<TN>;
    using S = Sched<TN>;
    constexpr int FI = T::FI, FJ = T::FJ, NW = S::NW;
    constexpr int WN = kNW / T::WM;
    constexpr bool kGate = EPI == PMA_EPI_GATE_RESIDUAL || EPI == kEpiGateStats;
    static_assert(TN == 256 || (TN == 224 && (EPI == PMA_EPI_STORE || kGate)) ||
                      (TN == 128 && (EPI == kEpiQkvF16 || EPI == kEpiQkvF8)),
                  "tile shapes: 224 for the store and gated residual, 128 for the QKV epilogue");
    // five 32 KB slots, each one operand half-stage (256 rows x 64 K): half h
    // (A of stage s is h = 2s, W of stage s is h = 2s + 1) lives in slot
    // (h + 2 P0) % 5, P0 the ring's phase offset below; one object per slot,
    // so the compiler can tell the slot being streamed into from the ones
    // being read
    __shared__ __attribute__((aligned(1024))) uint16_t h0[kStageElems];
    __shared__ __attribute__((aligned(1024))) uint16_t h1[kStageElems];
    __shared__ __attribute__((aligned(1024))) uint16_t h2[kStageElems];
    __shared__ __attribute__((aligned(1024))) uint16_t h3[kStageElems];
    __shared__ __attribute__((aligned(1024))) uint16_t h4[kStageElems];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int wm = wave / WN, wn = wave % WN;

    // ---- tiles (XCD-aware, grouped).  With the store and SwiGLU epilogues on
    // 256-wide tiles the workgroups are persistent: workgroup b runs the tiles
    // b/8, b/8 + G/8, ... of XCD b%8's share (G workgroups), and issues the
    // next tile's first DMA before the current tile's epilogue, whose stores
    // then overlap the next tile's first stages.  (The gated residual reads R
    // and the gate in its epilogue, loads that would wait behind that DMA:
    // 0.5-2% slower persistent, as were the 224-wide store tiles; the QKV
    // epilogue uses the LDS.)
    constexpr bool kPersist = TN == 256 && (EPI == PMA_EPI_STORE || EPI == PMA_EPI_SWIGLU);
    const int tiles_m = (a.M + kTM - 1) / kTM;
    const int out_tn = (EPI == PMA_EPI_SWIGLU) ? TN / 2 : TN;
    const int tiles_n = (a.n_end - a.n_begin) / out_tn;   // output columns [n_begin, n_end)
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + 7) / 8;
    const int xcd = (int)(blockIdx.x & 7);
    int li = (int)(blockIdx.x >> 3);
    if (li >= per_xcd || xcd * per_xcd + li >= total) return;
    const int per_group = kGroupM * tiles_n;
    auto tile_of = [&](int l, int &tm0, int &tn0) __attribute__((always_inline)) {
        const int t = xcd * per_xcd + l;
        const int group = t / per_group;
        const int first_m = group * kGroupM;
        const int gsize = min(kGroupM, tiles_m - first_m);
        tm0 = (first_m + (t % per_group) % gsize) * kTM;
        tn0 = a.n_begin + ((t % per_group) / gsize) * out_tn;
    };
    int m0, n0;
    tile_of(li, m0, n0);

    // ---- operand streams.  A rows m0.. (bound: rows < M), W rows from the
    // tile's first (the SwiGLU up rows N further on); offsets are relative to
    // the tile's rows, so only the buffer resources change from tile to tile.
    auto a_rsrc = [&](int tm0) __attribute__((always_inline)) {
        return make_rsrc(a.A + (int64_t)tm0 * a.lda, (uint32_t)(a.M - tm0) * (uint32_t)a.lda * 2u);
    };
    auto w_rsrc = [&](int tn0) __attribute__((always_inline)) {
        return make_rsrc(a.W + (int64_t)tn0 * a.ldw, a.w_bytes - (uint32_t)tn0 * (uint32_t)a.ldw * 2u);
    };
    __amdgpu_buffer_rsrc_t ars = a_rsrc(m0), wrs = w_rsrc(n0);
    // wave-instruction j of a half fills tile rows 8j..8j+7 (lane l: row
    // 8j + l/8, position l%8, fetching the chunk the swizzle places there);
    // this wave issues j = 8*wave + i (A) and j = NW*wave + i (W) of every
    // half.  Halves past the last stage re-read the last one (into a slot no
    // wave reads again), so every stage issues the same DMA instructions.
    uint32_t avo[8], wvo[NW];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 8 * (8 * wave + i) + (lane >> 3), c = g_pos(r, lane & 7);
        avo[i] = 2u * ((uint32_t)r * (uint32_t)a.lda + 8u * c);
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int r = 8 * (NW * wave + i) + (lane >> 3), c = g_pos(r, lane & 7);
        int wrow;
        if (EPI == PMA_EPI_SWIGLU) {
            // W-tile rows 64w..64w+63 = [gate 32w..32w+31 | up 32w..32w+31]
            const int w = r >> 6, rr = r & 63;
            wrow = 32 * w + (rr & 31) + ((rr & 32) ? a.N : 0);
        } else {
            wrow = r;
        }
        wvo[i] = 2u * ((uint32_t)wrow * (uint32_t)a.ldw + 8u * c);
    }
    const int nk = a.K / kTK;   // >= 1, nk % 5 == R

    auto slot = [&](int s) __attribute__((always_inline)) -> uint16_t * {
        s %= 5;
        return s == 0 ? h0 : s == 1 ? h1 : s == 2 ? h2 : s == 3 ? h3 : h4;
    };
    // interval position q of the interval that ends at stage st's barrier: W
    // half of stage st+1 (q < NW), then A half of stage st+2.  P: st % 5,
    // known at compile time.
    auto dma_q = [&](int st, int P, int q) __attribute__((always_inline)) {
        if (q < NW) {
            const uint32_t so = 2u * (uint32_t)(min(st + 1, nk - 1) * kTK);
            dma16(wrs, (lds_void *)&slot(2 * P + 3)[(NW * wave + q) * 512], wvo[q], so);
        } else {
            const uint32_t so = 2u * (uint32_t)(min(st + 2, nk - 1) * kTK);
            dma16(ars, (lds_void *)&slot(2 * P + 4)[(8 * wave + q - NW) * 512], avo[q - NW], so);
        }
    };

    f32x16 acc[FI][FJ];

    // fragment rows of this lane in the two tiles; fragments of a k-step (16
    // deep) are read one k-step ahead of their MFMAs, across stage ends too,
    // in the order the MFMAs first use them
    const int arow0 = (kTM / T::WM) * wm + l32, wrow0 = (TN / WN) * wn + l32;
    bf16x8 af[2][FI], wf[2][FJ];
    auto load_frags = [&](const uint16_t *at, const uint16_t *wt, int kk, bf16x8 (&fa)[FI],
                          bf16x8 (&fw)[FJ]) __attribute__((always_inline)) {
        fa[0] = *reinterpret_cast<const bf16x8 *>(at + arow0 * kTK + 8 * g_pos(arow0, 2 * kk + hi));
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int q = wrow0 + 32 * j;
            fw[j] = *reinterpret_cast<const bf16x8 *>(wt + q * kTK + 8 * g_pos(q, 2 * kk + hi));
        }
#pragma unroll
        for (int i = 1; i < FI; ++i) {
            const int r = arow0 + 32 * i;
            fa[i] = *reinterpret_cast<const bf16x8 *>(at + r * kTK + 8 * g_pos(r, 2 * kk + hi));
        }
    };
    // FI*FJ MFMAs, with the FI+FJ fragment reads of the next k-step and n DMA
    // instructions (positions q0.. of interval st) interleaved evenly
    auto mfmas = [&](bf16x8 (&fa)[FI], bf16x8 (&fw)[FJ], int st, int P, int q0, int n)
                     __attribute__((always_inline)) {
        constexpr int nM = FI * FJ, nR = FI + FJ;
        static_assert(nR <= nM, "at most one fragment read after each MFMA");
#pragma unroll
        for (int q = 0; q < n; ++q) dma_q(st, P, q0 + q);
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[j], fa[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < nM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (((i + 1) * nR + nM - 1) / nM != (i * nR + nM - 1) / nM)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if ((i * n) / nM != ((i + 1) * n) / nM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };

    // Stage st (phase P = st % 5): its halves sit in slots 2P and 2P+1 (mod 5).
    // Its four k-steps read their fragments one k-step ahead.  After the
    // MFMAs of k-step 2 every wave has its k-step 3 fragments in registers;
    // the wait there leaves only the A half of stage st+2 in flight (the W
    // half of st+1 landed), and the barrier makes stage st+1 readable (k-step
    // 3 reads its first fragments) and frees both slots of stage st: the W
    // half of st+2 (k-step 3 on) and the A half of st+3 (next stage) go there.
    auto stage = [&](int st, int P) __attribute__((always_inline)) {
        const uint16_t *ca = slot(2 * P), *cw = slot(2 * P + 1);
#pragma unroll
        for (int kk = 0; kk < 3; ++kk) {
            load_frags(ca, cw, kk + 1, af[(kk + 1) & 1], wf[(kk + 1) & 1]);
            mfmas(af[kk & 1], wf[kk & 1], st, P, S::first(kk + 1), S::n[kk + 1]);
        }
        // this wave's DMA instructions, all but the interval's A half, landed
        __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (0 << 8));   // vmcnt(8) lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        load_frags(slot(2 * P + 2), slot(2 * P + 3), 0, af[0], wf[0]);
        mfmas(af[1], wf[1], st + 1, P + 1, 0, S::n[0]);
    };

    // ---- the ring's phase: stage st has phase (st + P0) % 5.  With 256- and
    // 128-wide tiles the first H stages (H = R, or a whole period when R = 0) run ahead
    // of the unrolled loop, ending at phase 4, and the loop runs whole periods
    // from phase 0: after a remainder placed behind the loop the compiler moved
    // the accumulators between registers (about 3600 moves per tile, 1.5% of
    // the kernel's time at R = 4).  The 224-wide tiles keep the remainder behind
    // the loop, where they measured 2% faster.
    constexpr bool kHeadPeel = TN != 224;
    constexpr int H = !kHeadPeel ? 0 : R == 0 ? 5 : R;
    constexpr int P0 = (5 - H) % 5;
    // ---- prologue: stages 0 and the A half of 1 requested and the leading
    // part of the W half of 1 (what k-step 3 of a stage -1 would issue)
    auto prologue = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) dma16(ars, (lds_void *)&slot(2 * P0)[(8 * wave + i) * 512], avo[i], 0u);
#pragma unroll
        for (int i = 0; i < NW; ++i)
            dma16(wrs, (lds_void *)&slot(2 * P0 + 1)[(NW * wave + i) * 512], wvo[i], 0u);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dma16(ars, (lds_void *)&slot(2 * P0 + 2)[(8 * wave + i) * 512], avo[i],
                  2u * (uint32_t)(min(1, nk - 1) * kTK));
#pragma unroll
        for (int q = 0; q < S::n[0]; ++q) dma_q(0, P0, q);
    };
    prologue();
    for (;;) {
    // stage 0 landed
    PMA_STAGE_END(8 + S::n[0]);
    load_frags(slot(2 * P0), slot(2 * P0 + 1), 0, af[0], wf[0]);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    if constexpr (H > 0) stage(0, P0);
    if constexpr (H > 1) stage(1, P0 + 1);
    if constexpr (H > 2) stage(2, P0 + 2);
    if constexpr (H > 3) stage(3, P0 + 3);
    if constexpr (H > 4) stage(4, P0 + 4);
    int st = H;
    for (; st + 5 <= nk; st += 5) {
        stage(st, 0);
        stage(st + 1, 1);
        stage(st + 2, 2);
        stage(st + 3, 3);
        stage(st + 4, 4);
    }
    if constexpr (!kHeadPeel) {
        if constexpr (R > 0) stage(st, 0);
        if constexpr (R > 1) stage(st + 1, 1);
        if constexpr (R > 2) stage(st + 2, 2);
        if constexpr (R > 3) stage(st + 3, 3);
    }
    // no DMA may still be writing when the slots are reused or released
    PMA_STAGE_END(0);
    // the next tile's first DMA goes out before this tile's epilogue (which
    // does not use the LDS)
    const int cm0 = m0, cn0 = n0;
    bool more = false;
    if constexpr (kPersist) {
        li += (int)(gridDim.x >> 3);
        more = li < per_xcd && xcd * per_xcd + li < total;
        if (more) {
            tile_of(li, m0, n0);
            ars = a_rsrc(m0);
            wrs = w_rsrc(n0);
            prologue();
        }
    }

    // ---- epilogue.  acc[i][j] register v: output row m0 + (256/WM)*wm + 32*i + l32,
    // W-tile row (TN/WN)*wn + 32*j + 8*(v/4) + 4*hi + v%4.
    if constexpr (EPI == kEpiQkvF16 || EPI == kEpiQkvF8) {
        // the ring is free again (every wave is past the last stage's barrier)
        uint16_t *stg = wave == 0 ? h0 : wave == 1 ? h1 : wave == 2 ? h2 : h3;
        qkv_epilogue<EPI == kEpiQkvF16 ? 16 : 8, FI>(a, acc, cm0, cn0, wm, wn, l32, hi, stg);
        return;
    }
#pragma unroll
    for (int i = 0; i < FI; ++i) {
        const int m = cm0 + (kTM / T::WM) * wm + 32 * i + l32;
        if (m >= a.M) continue;
        uint16_t *crow = a.C + (int64_t)m * a.ldc;
        if constexpr (EPI == PMA_EPI_SWIGLU) {
            // W-tile rows 128 wn + 64 jj + [0, 64) are the gate rows (acc[i][2 jj])
            // and the up rows (acc[i][2 jj + 1]) of outputs n0 + 32 (2 wn + jj) + [0, 32)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = cn0 + 32 * (2 * wn + jj) + 8 * g + 4 * hi;
                    float h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        h[e] = silu(acc[i][2 * jj][4 * g + e]) * acc[i][2 * jj + 1][4 * g + e];
                    uint2 w;
                    w.x = pack_bf16x2(h[0], h[1]);
                    w.y = pack_bf16x2(h[2], h[3]);
                    *reinterpret_cast<uint2 *>(crow + col) = w;
                }
        } else {
            const float *grow = nullptr;
            const uint16_t *rrow = nullptr;
            if (kGate) {
                const int tag = a.tags[m], ts = a.ts_idx[m];
                rrow = a.R + (int64_t)m * a.ldr;
                // rows outside the table (padding, or an index a layout check
                // would reject) take a zero gate
                if (tag >= 0 && tag <= 2 && (uint32_t)ts < (uint32_t)a.T)
                    grow = a.table + ((int64_t)(tag * a.T + ts) * 6 + a.gate_chunk) * a.N;
            }
#pragma unroll
            for (int j = 0; j < FJ; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = cn0 + (TN / WN) * wn + 32 * j + 8 * g + 4 * hi;
                    float y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e];
                    if (kGate) {
                        const uint2 rv = *reinterpret_cast<const uint2 *>(rrow + col);
                        float r4[4] = {bf16_bits_to_f32(rv.x & 0xffff), bf16_bits_to_f32(rv.x >> 16),
                                       bf16_bits_to_f32(rv.y & 0xffff), bf16_bits_to_f32(rv.y >> 16)};
                        f32x4 gv = {0.f, 0.f, 0.f, 0.f};
                        if (grow) gv = *reinterpret_cast<const f32x4 *>(grow + col);
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = r4[e] + gv[e] * y[e];
                    }
                    uint2 w;
                    w.x = pack_bf16x2(y[0], y[1]);
                    w.y = pack_bf16x2(y[2], y[3]);
                    *reinterpret_cast<uint2 *>(crow + col) = w;
                    if constexpr (EPI == kEpiGateStats) {
                        // keep the rounded values (what the next norm reads)
                        acc[i][j][4 * g] = bf16_bits_to_f32(w.x & 0xffff);
                        acc[i][j][4 * g + 1] = bf16_bits_to_f32(w.x >> 16);
                        acc[i][j][4 * g + 2] = bf16_bits_to_f32(w.y & 0xffff);
                        acc[i][j][4 * g + 3] = bf16_bits_to_f32(w.y >> 16);
                    }
                }
            if constexpr (EPI == kEpiGateStats) {
                // the row's TN / WN columns of this wave: FJ * 16 in this lane,
                // as many in lane l ^ 32.  Mean first, then the squared
                // deviations from it (four independent chains each).
                constexpr int GW = TN / WN;
                float c4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) c4[v & 3] += acc[i][j][v];
                const float mean = pair_sum((c4[0] + c4[1]) + (c4[2] + c4[3])) * (1.0f / GW);
                float q4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const float d = acc[i][j][v] - mean;
                        q4[v & 3] = fmaf(d, d, q4[v & 3]);
                    }
                const float m2 = pair_sum((q4[0] + q4[1]) + (q4[2] + q4[3]));
                if (hi == 0)
                    a.stats[(int64_t)m * a.stats_groups + (cn0 - a.n_begin) / GW + wn] = make_float2(mean, m2);
            }
        }
    }
    if (!more) break;
    }
}

template <int EPI, int TN>
void launch_r(const GemmLaunch &a, dim3 grid, int nt, hipStream_t s) {
    switch ((a.K / kTK) % 5) {
        case 0: gemm_kernel<EPI, 0, TN><<<grid, nt, 0, s>>>(a); break;
        case 1: gemm_kernel<EPI, 1, TN><<<grid, nt, 0, s>>>(a); break;
        case 2: gemm_kernel<EPI, 2, TN><<<grid, nt, 0, s>>>(a); break;
        case 3: gemm_kernel<EPI, 3, TN><<<grid, nt, 0, s>>>(a); break;
        default: gemm_kernel<EPI, 4, TN><<<grid, nt, 0, s>>>(a); break;
    }
}

int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace

int gemm_tile_n(int epi, int M, int N) {
    if ((epi != PMA_EPI_STORE && epi != PMA_EPI_GATE_RESIDUAL && epi != kEpiGateStats) || N % 224 != 0)
        return 256;
    // rounds of tiles over the CUs, each round as long as its tiles are wide;
    // the narrower tile is taken when it saves at least 5%
    const int64_t cus = device_cus();
    const int64_t tiles_m = (M + kTM - 1) / kTM;
    const int64_t r256 = (tiles_m * (N / 256) + cus - 1) / cus;
    const int64_t r224 = (tiles_m * (N / 224) + cus - 1) / cus;
    return r224 * 224 * 100 < r256 * 256 * 95 ? 224 : 256;
}

int gemm_stats_group_width(int M, int N) {
    // a wave of a 224-wide tile holds a row's 224 columns; of a 256-wide
    // tile (2 x 2 waves), 128 of them
    return gemm_tile_n(kEpiGateStats, M, N) == 224 ? 224 : 128;
}

int gemm_qkv_narrow_columns(int M, int N) {
    // The QKV projection's 256-wide column tiles, the last k of them run as
    // 128-wide tiles (twice as many, each about 0.6 of a wide tile's time) in
    // a second launch, when that shortens a problem of two or more rounds by
    // at least 3%: at M = 8192, N = 21504 the 2688 wide tiles are 10.5 rounds
    // on 256 CUs; 2560 wide + 256 narrow tiles are 10 rounds + one narrow one.
    const int64_t cus = device_cus();
    const int64_t tiles_m = (M + kTM - 1) / kTM, tn = N / 256;
    auto est = [&](int64_t k) {
        return 10 * ((tiles_m * (tn - k) + cus - 1) / cus) + 6 * ((2 * k * tiles_m + cus - 1) / cus);
    };
    const int64_t base = est(0);
    if (base < 20) return 0;
    int64_t best = 0, best_t = base;
    for (int64_t k = 1; k <= tn; ++k)
        if (est(k) < best_t) best = k, best_t = est(k);
    return best_t * 100 <= base * 97 ? (int)(best * 256) : 0;
}

namespace {

template <int EPI, int TN>
void launch_cols(const GemmLaunch &a, int n_begin, int n_end, hipStream_t s) {
    GemmLaunch b = a;
    b.n_begin = n_begin;
    b.n_end = n_end;
    const int tiles_m = (b.M + kTM - 1) / kTM;
    const int out_tn = (EPI == PMA_EPI_SWIGLU) ? TN / 2 : TN;
    const int total = tiles_m * ((n_end - n_begin) / out_tn);
    const int per_xcd = (total + 7) / 8;
    // persistent epilogues: one workgroup per CU (the LDS admits one)
    const bool persist = TN == 256 && (EPI == PMA_EPI_STORE || EPI == PMA_EPI_SWIGLU);
    const int per_xcd_wg = persist ? min(per_xcd, max(1, device_cus() / 8)) : per_xcd;
    launch_r<EPI, TN>(b, dim3(8 * per_xcd_wg), kNW * 64, s);
}

template <int EPI>
void launch_qkv(const GemmLaunch &a, hipStream_t s) {
    const int narrow = gemm_qkv_narrow_columns(a.M, a.N);
    if (narrow < a.N) launch_cols<EPI, 256>(a, 0, a.N - narrow, s);
    if (narrow > 0) launch_cols<EPI, 128>(a, a.N - narrow, a.N, s);
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch &a, hipStream_t s) {
    const int tn = gemm_tile_n(a.epi, a.M, a.N);
    switch (a.epi) {
        case PMA_EPI_STORE:
            if (tn == 224) launch_cols<PMA_EPI_STORE, 224>(a, 0, a.N, s);
            else launch_cols<PMA_EPI_STORE, 256>(a, 0, a.N, s);
            break;
        case PMA_EPI_GATE_RESIDUAL:
            if (tn == 224) launch_cols<PMA_EPI_GATE_RESIDUAL, 224>(a, 0, a.N, s);
            else launch_cols<PMA_EPI_GATE_RESIDUAL, 256>(a, 0, a.N, s);
            break;
        case kEpiGateStats:
            if (tn == 224) launch_cols<kEpiGateStats, 224>(a, 0, a.N, s);
            else launch_cols<kEpiGateStats, 256>(a, 0, a.N, s);
            break;
        case PMA_EPI_SWIGLU: launch_cols<PMA_EPI_SWIGLU, 256>(a, 0, a.N, s); break;
        case kEpiQkvF16: launch_qkv<kEpiQkvF16>(a, s); break;
        case kEpiQkvF8: launch_qkv<kEpiQkvF8>(a, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pma
