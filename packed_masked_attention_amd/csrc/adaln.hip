// adaln.hip -- AdaLN modulation table: table[g][t][k][c] = temb[t] . W_ada[g][k*hidden + c].
//
// Page "MiniMaxH3Transformer3DModel" (diffusers API page): constructor
// parameters -- time_embed_dim is the output of the timestep MLP and the
// input of every AdaLN projection; intro -- the per-row modality tag selects
// the modulation parameters.  Reading: one linear map per tag g (0 video,
// 1 text, 2 audio) from time_embed_dim to 6 * hidden, no bias; the six
// chunks are shift_a, scale_a, gate_a, shift_f, scale_f, gate_f.
//
// A skinny GEMM (T distinct timesteps x 3*6*hidden outputs) bound by reading
// the 3 x 6*hidden x E bf16 weights once: 16 lanes per weight row read it in
// 16-byte chunks, four in flight per lane and nontemporal (read once: 89.9 ->
// 79.6 us for 520 MB, 6.5 TB/s); the T embeddings sit in LDS; fp32
// accumulation.
#include "internal.h"

namespace pma {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxT = 8;

__global__ __launch_bounds__(kThreads) void adaln_table_kernel(AdaLnLaunch a) {
    extern __shared__ uint16_t temb_s[];   // [T][E] bf16
    const int n_e = a.T * a.E;
    for (int i = threadIdx.x * 8; i < n_e; i += kThreads * 8)
        *reinterpret_cast<u16x8 *>(temb_s + i) = *reinterpret_cast<const u16x8 *>(a.temb + i);
    __syncthreads();
    const int grp = threadIdx.x >> 4, gl = threadIdx.x & 15;
    const int64_t rows = 3ll * 6 * a.hidden;
    const int64_t r = (int64_t)blockIdx.x * (kThreads / 16) + grp;
    if (r >= rows) return;
    const uint16_t *w = a.w + r * a.E;
    float acc[kMaxT];
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) acc[t] = 0.f;
#pragma unroll 4
    for (int e = gl * 8; e < a.E; e += 128) {
        const u16x8 wr = __builtin_nontemporal_load(reinterpret_cast<const u16x8 *>(w + e));
        float wf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) wf[j] = bf16_bits_to_f32(wr[j]);
#pragma unroll
        for (int t = 0; t < kMaxT; ++t) {
            if (t < a.T) {
                const u16x8 te = *reinterpret_cast<const u16x8 *>(temb_s + t * a.E + e);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[t] = fmaf(wf[j], bf16_bits_to_f32(te[j]), acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
        float v = acc[t];
        v += __shfl_xor(v, 1, 16);
        v += __shfl_xor(v, 2, 16);
        v += __shfl_xor(v, 4, 16);
        v += __shfl_xor(v, 8, 16);
        acc[t] = v;
    }
    // row r = g * 6*hidden + k*hidden + c  ->  table[g][t][k][c]
    const int64_t six_h = 6ll * a.hidden;
    const int64_t g = r / six_h, kc = r % six_h;
    if (gl < kMaxT && gl < a.T) {
        float v = acc[0];
#pragma unroll
        for (int t = 1; t < kMaxT; ++t) if (gl == t) v = acc[t];
        a.table[(g * a.T + gl) * six_h + kc] = v;
    }
}

}  // namespace

hipError_t launch_adaln_table(const AdaLnLaunch &a, hipStream_t s) {
    const int64_t rows = 3ll * 6 * a.hidden;
    const int blocks = (int)((rows + 15) / 16);
    adaln_table_kernel<<<blocks, kThreads, (size_t)a.T * a.E * 2, s>>>(a);
    return hipGetLastError();
}

int adaln_max_t() { return kMaxT; }

}  // namespace pma
