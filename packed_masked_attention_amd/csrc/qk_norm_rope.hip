// qk_norm_rope.hip -- per-head QK-RMSNorm + 3-axis RoPE, and the relayout of
// Q, K, V into the flash attention kernel's operands.
//
// Page "MiniMaxH3Transformer3DModel" (diffusers API page), constructor
// parameters: qk_norm_eps of the per-head query/key norms; rope_freq_dim F
// frequencies per axis, one inv_freq buffer shared by the t, h and w axes,
// 2*3*F rotated channels; rope_theta the base of the frequency schedule.
// Page "MiniMax H3 Inference Engine voor Mac computers", checkpoint layout
// notes: the QK normalisation and RoPE run as one fused kernel.
//
// Readings: RMSNorm over the head's 128 channels with one fp32 weight vector
// shared by all heads; inv_freq[f] = theta^(-f/F); axis a rotates channel
// pairs (2aF+f, 2aF+f+F) by (pos[a]*pos_scale[a])*inv_freq[f] (rotate-half
// pairing, direction e^{+i phi}); channels >= 6F pass through.  The per-axis
// scale is 1 except where the caller asks otherwise (the engine page's
// 256x256 preview halves the spatial coordinates).
//
// Q' leaves multiplied by qscale (softmax_scale * log2 e): the attention
// kernel then reads log2-unit logits straight out of its QK product.
//
// HBM-bound: per (row, head) it reads 3 x 256 B and writes 3 x 256 B.
// Block = 64 rows x 4 heads.  The block's V loads (16 per thread) are issued
// first and stay in flight through the rest.  Each 16-lane group owns one
// (row, head) of Q or K, 8 channels (16 bytes) per lane, and keeps eight
// such items' loads in flight before it computes them; the sum of squares is
// reduced across the group and the RoPE partner channels c +/- F sit F/8
// lanes away, both exchanged by DPP moves inside the 16-lane row.  cos/sin of
// the 64 rows x 3F angles are computed once per block in fp64 (angles reach
// ~1e3 rad, so no fast-math approximation) and kept in LDS as fp32.  V goes
// through LDS and leaves transposed, keys contiguous per (head, channel).
// Every input is read once and every output written once, so loads and stores
// are nontemporal (streamed past the caches: 325 -> 298 us at L = 16384, 56
// heads, bit-identical output).
#include "internal.h"

namespace pma {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 64;      // rows per block
constexpr int kHeads = 4;      // heads per block
constexpr int kThreads = 256;
constexpr int kVRow = kHeadDim + 2;  // LDS row of the V tile in bf16: 65 words, so the
                                     // transposed 2-byte reads spread over the banks

// Cross-lane moves inside a 16-lane row on the VALU (DPP), without the LDS
// crossbar: lane i reads lane i^1, i^2 (quad permutes) or (i+4)%16, (i+8)%16
// (row rotations).
__device__ __forceinline__ float dpp_f(float x, int ctrl_sel) {
    const int v = __float_as_int(x);
    int r;
    switch (ctrl_sel) {
        case 1: r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
        case 2: r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
        case 4: r = __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false); break;  // row_ror:4
        default: r = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false); break; // row_ror:8
    }
    return __int_as_float(r);
}

template <int F>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(PrepLaunch a) {
    __shared__ float2 cs[kRows][48];                    // (cos, sin) per row, axis*F + f
    __shared__ uint32_t vtile32[kRows * kVRow / 2];
    uint16_t *vtile = reinterpret_cast<uint16_t *>(vtile32);

    const int tid = threadIdx.x;
    const int r0 = blockIdx.x * kRows;
    const int h0 = blockIdx.y * kHeads;
    const int nh = min(kHeads, a.H - h0);
    const int nang = 3 * F;

    // ---- V loads of every head first: they stay in flight through the
    // table and the Q/K work
    u16x8 vraw[kHeads][kRows * 16 / kThreads];
#pragma unroll
    for (int hl = 0; hl < kHeads; ++hl)
#pragma unroll
        for (int k = 0; k < kRows * 16 / kThreads; ++k) {
            const int e = tid + k * kThreads;
            const int rl = e / 16, c8 = e % 16;
            const int row = r0 + rl;
            vraw[hl][k] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (hl < nh && row < a.L)
                vraw[hl][k] = __builtin_nontemporal_load(reinterpret_cast<const u16x8 *>(a.v + (int64_t)row * a.v_ld +
                                                               (h0 + hl) * kHeadDim + c8 * 8));
        }

    // ---- cos/sin table of this block's rows
    for (int e = tid; e < kRows * nang; e += kThreads) {
        const int rl = e / nang, j = e % nang;
        const int row = r0 + rl;
        float c = 1.f, s = 0.f;
        if (row < a.L) {
            const int ax = j / F, f = j % F;
            const double phi = ((double)a.pos[3 * (int64_t)row + ax] * a.pos_scale[ax]) * a.inv_freq[f];
            double sd, cd;
            sincos(phi, &sd, &cd);
            c = (float)cd;
            s = (float)sd;
        }
        cs[rl][j] = make_float2(c, s);
    }
    __syncthreads();

    // ---- Q and K: items (tensor, head, row) with rows fastest, 16 lanes each
    const int chunk = tid & 15;          // channels 8*chunk .. 8*chunk+7
    const int sub = tid >> 4;            // 16 items per pass
    const int n_items = 2 * nh * kRows;
    const int sec_chunks = F / 4;        // chunks per rotated section (2F channels)
    const int half_chunks = F / 8;       // chunk distance of the partner channel
    const bool rotated = chunk < 3 * sec_chunks;
    const int ax = rotated ? chunk / sec_chunks : 0;
    const int in_sec = chunk % sec_chunks;
    const bool first_half = in_sec < half_chunks;
    const int f0 = (first_half ? in_sec : in_sec - half_chunks) * 8;
    constexpr int kB = 8;   // items in flight per 16-lane group
    for (int base = sub; base < n_items; base += kB * (kThreads / 16)) {
        u16x8 raw[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int item = base + u * (kThreads / 16);
            const int rl = item % kRows;
            const int hl = (item / kRows) % nh;
            const int tensor = item / (kRows * nh);
            const int row = r0 + rl;
            const uint16_t *src = tensor ? a.k : a.q;
            const int64_t ld = tensor ? a.k_ld : a.q_ld;
            raw[u] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (item < n_items && row < a.L)
                raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u16x8 *>(src + (int64_t)row * ld +
                                                          (h0 + hl) * kHeadDim + chunk * 8));
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int item = base + u * (kThreads / 16);
            if (item >= n_items) break;
            const int rl = item % kRows;
            const int hl = (item / kRows) % nh;
            const int tensor = item / (kRows * nh);   // 0 = Q, 1 = K
            const int row = r0 + rl;
            const int h = h0 + hl;
            const float *w = tensor ? a.wk : a.wq;
            uint16_t *dst = tensor ? a.kh : a.qh;
            float x[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] = bf16_bits_to_f32(raw[u][t]);
            float ss = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) ss = fmaf(x[t], x[t], ss);
            // all 16 lanes end with the group's sum: pairs, quads, then the
            // quad sums rotated in by 4 and 8
            ss += dpp_f(ss, 1);
            ss += dpp_f(ss, 2);
            ss += dpp_f(ss, 4);
            ss += dpp_f(ss, 8);
            // Q' also carries the attention's logit scale
            const float r = (tensor ? 1.0f : a.qscale) / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
            const f32x4 w0 = *reinterpret_cast<const f32x4 *>(w + chunk * 8);
            const f32x4 w1 = *reinterpret_cast<const f32x4 *>(w + chunk * 8 + 4);
            float n[8];
            n[0] = x[0] * r * w0[0]; n[1] = x[1] * r * w0[1];
            n[2] = x[2] * r * w0[2]; n[3] = x[3] * r * w0[3];
            n[4] = x[4] * r * w1[0]; n[5] = x[5] * r * w1[1];
            n[6] = x[6] * r * w1[2]; n[7] = x[7] * r * w1[3];
            float y[8];
            // partner channels: chunk +/- F/8 within the 16-lane group
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                // partner channel: F/8 chunks away, i.e. lane ^ 1 (F = 8) or ^ 2 (F = 16)
                const float pn = dpp_f(n[t], half_chunks);
                if (rotated) {
                    const float2 e = cs[rl][ax * F + f0 + t];
                    y[t] = first_half ? (n[t] * e.x - pn * e.y) : (n[t] * e.x + pn * e.y);
                } else {
                    y[t] = n[t];
                }
            }
            uint32_t packed[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) packed[t] = pack_bf16x2(y[2 * t], y[2 * t + 1]);
            u32x4 out = {packed[0], packed[1], packed[2], packed[3]};
            if (row >= a.L) out = u32x4{0, 0, 0, 0};
            __builtin_nontemporal_store(out, reinterpret_cast<u32x4 *>(dst + ((int64_t)h * a.Lp + row) * kHeadDim + chunk * 8));
        }
    }

    // ---- V: stage [64 rows][128] per head, write [128 channels][64 rows]
#pragma unroll
    for (int hl = 0; hl < kHeads; ++hl) {
        if (hl >= nh) break;
        const int h = h0 + hl;
#pragma unroll
        for (int k = 0; k < kRows * 16 / kThreads; ++k) {
            const int e = tid + k * kThreads;
            const int rl = e / 16, c8 = e % 16;
            const uint4 w4 = __builtin_bit_cast(uint4, vraw[hl][k]);
            uint32_t *d32 = vtile32 + (rl * kVRow + c8 * 8) / 2;
            d32[0] = w4.x; d32[1] = w4.y; d32[2] = w4.z; d32[3] = w4.w;
        }
        __syncthreads();
        // 128 channels x 8 row-groups of 8 rows; 8 consecutive lanes cover one
        // channel's 64 rows (128 contiguous bytes)
        for (int e = tid; e < kHeadDim * 8; e += kThreads) {
            const int g = e % 8, c = e / 8;
            u16x8 col;
#pragma unroll
            for (int t = 0; t < 8; ++t) col[t] = vtile[(g * 8 + t) * kVRow + c];
            __builtin_nontemporal_store(col, reinterpret_cast<u16x8 *>(a.vt + ((int64_t)h * kHeadDim + c) * a.Lp + r0 + g * 8));
        }
        __syncthreads();
    }
}

// One thread per (row, angle): the same fp64 angle and sincos as the table
// above, stored as fp32 for the fused QKV projection's epilogue.
__global__ __launch_bounds__(256) void rope_table_kernel(PrepLaunch a, float2 *rope) {
    const int nang = 3 * a.F;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)a.L * nang) return;
    const int row = (int)(e / nang), j = (int)(e % nang);
    const int ax = j / a.F, f = j % a.F;
    const double phi = ((double)a.pos[3 * (int64_t)row + ax] * a.pos_scale[ax]) * a.inv_freq[f];
    double sd, cd;
    sincos(phi, &sd, &cd);
    rope[e] = make_float2((float)cd, (float)sd);
}

}  // namespace

hipError_t launch_rope_table(const PrepLaunch &a, float2 *rope, hipStream_t s) {
    const int64_t n = (int64_t)a.L * 3 * a.F;
    rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a, rope);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const PrepLaunch &a, hipStream_t s) {
    dim3 grid(a.Lp / kRows, (a.H + kHeads - 1) / kHeads);
    if (a.F == 16)
        qk_norm_rope_kernel<16><<<grid, kThreads, 0, s>>>(a);
    else
        qk_norm_rope_kernel<8><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace pma
