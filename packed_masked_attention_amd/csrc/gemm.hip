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
// 128 gate rows + 128 up rows of W), K in steps of 64, eight waves (two per
// SIMD) in a 2 x 4 grid each owning a 128 x 64 block as 4 x 2 MFMA
// 32x32x16 tiles, so the 128 fp32 accumulators stay in VGPRs.  The MFMA
// computes D = W A^T (weights as the A operand), so a lane's accumulator
// column is one output ROW: per-row epilogue data (tag, timestep, residual
// row) is lane-constant and each lane writes runs of 4 consecutive bf16.
// Both operand tiles stream into LDS with buffer_load ... lds (rows past M
// read as zero through the buffer bound), double-buffered, 16-byte chunks
// XOR-swizzled by row so the fragment reads are bank-conflict-free.  Tiles
// are ordered in groups of 8 row-tiles and dealt out XCD-aware so each XCD
// works on a compact region sharing A and W panels in its L2.
#include "internal.h"

namespace pma {
namespace {

constexpr int kTM = 256;       // rows of A per tile
constexpr int kTN = 256;       // rows of W per tile
constexpr int kTK = 64;        // K per stage
constexpr int kTileElems = kTM * kTK;   // 16384 bf16 = 32 KB per operand tile
constexpr int kGroupM = 8;
constexpr int kRsrcFlags = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void;

// LDS position of 16-byte chunk c (0..7) of tile row r (128-byte rows).
__device__ __forceinline__ int g_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_void *l, uint32_t voff,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcFlags);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// QKV_ROPE epilogue ids: one per rope_freq_dim F (the partner of a rotated
// channel sits F/2 accumulator registers away in the same lane)
constexpr int kEpiQkvF16 = kEpiQkvRope;
constexpr int kEpiQkvF8 = kEpiQkvRope + 1;

// The QKV projection's epilogue.  The 256-column tile lies inside one of Q,
// K, V (H even) and holds two heads; wave (wm, wn) has tokens
// m0 + 128 wm + [0, 128) and channels 64 (wn & 1) + [0, 64) of head wn / 2.
// A lane's registers for one token: acc[i][j][v] = channel
// 64 (wn & 1) + 32 j + 8 (v / 4) + 4 hi + v % 4 of token m0 + 128 wm + 32 i + l32.
// Rows past the sequence have all-zero accumulators (their A rows read as
// zero), so the padding rows up to Lp come out as zeros.
template <int F>
__device__ __forceinline__ void qkv_epilogue(const GemmLaunch &a, f32x16 (&acc)[4][2], int m0,
                                             int n0, int wave, int wm, int wn, int l32, int hi,
                                             uint16_t *as0, uint16_t *as1, uint16_t *ws0,
                                             uint16_t *ws1) {
    const int HD = a.H * kHeadDim;
    const int tensor = n0 / HD;                        // 0 Q, 1 K, 2 V
    const int head = (n0 - tensor * HD) / kHeadDim + (wn >> 1);
    const int cb = 64 * (wn & 1);                      // the wave's first channel in the head
    if (tensor < 2) {
        // sum of squares per token: the lane's 32 channels, the other lane
        // half's 32, then the paired wave's 64 through LDS
        float *red = reinterpret_cast<float *>(as0);  // [8 waves][4][32]
        float ss[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) t = fmaf(acc[i][j][v], acc[i][j][v], t);
            const uint32_t u = __float_as_uint(t);
            const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            ss[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            if (hi == 0) red[(wave * 4 + i) * 32 + l32] = ss[i];
        }
        __syncthreads();
        const float *w = tensor ? a.wk : a.wq;
        uint16_t *dst = (tensor ? a.kh : a.qh) + (int64_t)head * a.Lp * kHeadDim;
        // the lane's 32 norm weights: channels cb + 32 j + 8 g + 4 hi + [0, 4)
        f32x4 wv[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                wv[j][g] = *reinterpret_cast<const f32x4 *>(w + cb + 32 * j + 8 * g + 4 * hi);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float tot = ss[i] + red[((wave ^ 1) * 4 + i) * 32 + l32];
            // Q' also carries the attention's logit scale
            const float rn = (tensor ? 1.0f : a.qscale) / sqrtf(tot * (1.0f / kHeadDim) + a.eps);
            const int m = m0 + 128 * wm + 32 * i + l32;
            // rows past the sequence are zero: any in-range table row serves
            const float2 *rope = a.rope + (int64_t)min(m, a.M - 1) * 3 * F;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float n[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) n[v] = acc[i][j][v] * rn * wv[j][v / 4][v % 4];
                float y[16];
                const int c0 = cb + 32 * j;             // first channel of this 32-channel run
                // registers v = 4 q + e hold channel c0 + 8 q + 4 hi + e; a group
                // of four is wholly rotated (c < 6F, four consecutive angles of
                // one section, partner F/2 registers away) or wholly passed on
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = c0 + 8 * q + 4 * hi;
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
                uint16_t *drow = dst + (int64_t)m * kHeadDim + c0 + 4 * hi;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint2 o;
                    o.x = pack_bf16x2(y[4 * g], y[4 * g + 1]);
                    o.y = pack_bf16x2(y[4 * g + 2], y[4 * g + 3]);
                    *reinterpret_cast<uint2 *>(drow + 8 * g) = o;
                }
            }
        }
    } else {
        // V^T: each wave stages its 64 channels x 128 tokens in its own 16 KB
        // of LDS, then writes 256-byte channel rows (tokens contiguous)
        uint16_t *st = (wave < 2 ? as0 : wave < 4 ? as1 : wave < 6 ? ws0 : ws1) + (wave & 1) * 8192;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int cl = 32 * j + 8 * (v / 4) + 4 * hi + v % 4;
                    st[cl * 128 + 32 * i + l32] = (uint16_t)(pack_bf16x2(acc[i][j][v], 0.f) & 0xffffu);
                }
        // the wave reads back only what it wrote; LDS keeps a wave's accesses in order
        const int lane = l32 + 32 * hi;
        uint16_t *vbase = a.vt + ((int64_t)head * kHeadDim + cb) * a.Lp + m0 + 128 * wm;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int row = it * 4 + (lane >> 4), ch = lane & 15;
            const uint4 val = *reinterpret_cast<const uint4 *>(st + row * 128 + ch * 8);
            *reinterpret_cast<uint4 *>(vbase + (int64_t)row * a.Lp + ch * 8) = val;
        }
    }
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_kernel(GemmLaunch a) {
    __shared__ __attribute__((aligned(1024))) uint16_t as0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t as1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t ws0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t ws1[kTileElems];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wm = wave >> 2, wn = wave & 3;

    // ---- tile (XCD-aware, grouped)
    const int tiles_m = (a.M + kTM - 1) / kTM;
    const int out_tn = (EPI == PMA_EPI_SWIGLU) ? kTN / 2 : kTN;
    const int tiles_n = a.N / out_tn;
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + 7) / 8;
    const int t = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (t >= total) return;
    const int per_group = kGroupM * tiles_n;
    const int group = t / per_group;
    const int first_m = group * kGroupM;
    const int gsize = min(kGroupM, tiles_m - first_m);
    const int tm = first_m + (t % per_group) % gsize;
    const int tn = (t % per_group) / gsize;
    const int m0 = tm * kTM;
    const int n0 = tn * out_tn;

    // ---- operand streams.  A rows m0.. (bound: rows < M), W rows per tile row.
    const uint32_t a_bytes = (uint32_t)(a.M - m0) * (uint32_t)a.lda * 2u;
    const __amdgpu_buffer_rsrc_t ars = make_rsrc(a.A + (int64_t)m0 * a.lda, a_bytes);
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(a.W, a.w_bytes);
    // wave-instruction j (0..31) fills tile rows 8j..8j+7; this wave issues j = 4*wave + i
    uint32_t avo[4], wvo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 4 * wave + i;
        const int r = 8 * j + (lane >> 3), p = lane & 7, c = g_pos(r, p);
        avo[i] = 2u * ((uint32_t)r * (uint32_t)a.lda + 8u * c);
        int wrow;
        if (EPI == PMA_EPI_SWIGLU) {
            // W-tile rows 64w..64w+63 = [gate 32w..32w+31 | up 32w..32w+31]
            const int w = r >> 6, rr = r & 63;
            wrow = n0 + 32 * w + (rr & 31) + ((rr & 32) ? a.N : 0);
        } else {
            wrow = n0 + r;
        }
        wvo[i] = 2u * ((uint32_t)wrow * (uint32_t)a.ldw + 8u * c);
    }
    auto dma = [&](int k0, uint16_t *ad, uint16_t *wd) __attribute__((always_inline)) {
        const uint32_t so = 2u * (uint32_t)k0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = 4 * wave + i;
            dma16(ars, (lds_void *)&ad[j * 512], avo[i], so);
            dma16(wrs, (lds_void *)&wd[j * 512], wvo[i], so);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // fragment rows of this lane in the two tiles
    const int arow0 = 128 * wm + l32, wrow0 = 64 * wn + l32;
    // one K-tile: four k-steps of 16; the fragments of step kk+1 are read
    // while step kk's 16 MFMAs run
    auto load_frags = [&](const uint16_t *at, const uint16_t *wt, int kk, bf16x8 (&af)[4],
                          bf16x8 (&wf)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = arow0 + 32 * i;
            af[i] = *reinterpret_cast<const bf16x8 *>(at + r * kTK + 8 * g_pos(r, 2 * kk + hi));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int q = wrow0 + 32 * j;
            wf[j] = *reinterpret_cast<const bf16x8 *>(wt + q * kTK + 8 * g_pos(q, 2 * kk + hi));
        }
    };
    auto compute = [&](const uint16_t *at, const uint16_t *wt) __attribute__((always_inline)) {
        bf16x8 af0[4], wf0[2], af1[4], wf1[2];
        load_frags(at, wt, 0, af0, wf0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 (&ac)[4] = (kk & 1) ? af1 : af0;
            bf16x8 (&wc)[2] = (kk & 1) ? wf1 : wf0;
            bf16x8 (&an)[4] = (kk & 1) ? af0 : af1;
            bf16x8 (&wn_)[2] = (kk & 1) ? wf0 : wf1;
            if (kk + 1 < 4) load_frags(at, wt, kk + 1, an, wn_);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wc[j], ac[i], acc[i][j],
                                                                        0, 0, 0);
            if (kk + 1 < 4) {
                __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }
        }
    };

    const int nk = a.K / kTK;
    dma(0, as0, ws0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        if (kt + 1 < nk) dma((kt + 1) * kTK, as1, ws1);
        compute(as0, ws0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < nk) {
            if (kt + 2 < nk) dma((kt + 2) * kTK, as0, ws0);
            compute(as1, ws1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    // ---- epilogue.  acc[i][j] register v: output row m0 + 128*wm + 32*i + l32,
    // W-tile row 64*wn + 32*j + 8*(v/4) + 4*hi + v%4.
    if constexpr (EPI == kEpiQkvF16 || EPI == kEpiQkvF8) {
        qkv_epilogue<EPI == kEpiQkvF16 ? 16 : 8>(a, acc, m0, n0, wave, wm, wn, l32, hi, as0, as1,
                                                  ws0, ws1);
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + 128 * wm + 32 * i + l32;
        if (m >= a.M) continue;
        uint16_t *crow = a.C + (int64_t)m * a.ldc;
        if (EPI == PMA_EPI_SWIGLU) {
            // acc[i][0] holds the gate rows of outputs n0 + 32*wn + [0,32),
            // acc[i][1] the matching up rows
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = n0 + 32 * wn + 8 * g + 4 * hi;
                    float h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        h[e] = silu(acc[i][0][4 * g + e]) * acc[i][1][4 * g + e];
                    uint2 w;
                    w.x = pack_bf16x2(h[0], h[1]);
                    w.y = pack_bf16x2(h[2], h[3]);
                    *reinterpret_cast<uint2 *>(crow + col) = w;
                }
        } else {
            const float *grow = nullptr;
            const uint16_t *rrow = nullptr;
            if (EPI == PMA_EPI_GATE_RESIDUAL) {
                const int tag = a.tags[m], ts = a.ts_idx[m];
                rrow = a.R + (int64_t)m * a.ldr;
                // rows outside the table (padding, or an index a layout check
                // would reject) take a zero gate
                if (tag >= 0 && tag <= 2 && (uint32_t)ts < (uint32_t)a.T)
                    grow = a.table + ((int64_t)(tag * a.T + ts) * 6 + a.gate_chunk) * a.N;
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = n0 + 64 * wn + 32 * j + 8 * g + 4 * hi;
                    float y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e];
                    if (EPI == PMA_EPI_GATE_RESIDUAL) {
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
                }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch &a, hipStream_t s) {
    const int tiles_m = (a.M + kTM - 1) / kTM;
    const int out_tn = (a.epi == PMA_EPI_SWIGLU) ? kTN / 2 : kTN;
    const int total = tiles_m * (a.N / out_tn);
    const int per_xcd = (total + 7) / 8;
    const dim3 grid(8 * per_xcd);
    switch (a.epi) {
        case PMA_EPI_STORE: gemm_kernel<PMA_EPI_STORE><<<grid, 512, 0, s>>>(a); break;
        case PMA_EPI_GATE_RESIDUAL:
            gemm_kernel<PMA_EPI_GATE_RESIDUAL><<<grid, 512, 0, s>>>(a);
            break;
        case PMA_EPI_SWIGLU: gemm_kernel<PMA_EPI_SWIGLU><<<grid, 512, 0, s>>>(a); break;
        case kEpiQkvF16: gemm_kernel<kEpiQkvF16><<<grid, 512, 0, s>>>(a); break;
        case kEpiQkvF8: gemm_kernel<kEpiQkvF8><<<grid, 512, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pma
