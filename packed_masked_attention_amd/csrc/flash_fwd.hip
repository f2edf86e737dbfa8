// flash_fwd.hip -- masked flash attention forward for gfx950 (bf16 MFMA).
//
// Page "MiniMaxH3Transformer3DModel" (diffusers API page): intro -- full
// self-attention over the packed sequence, padding rows (tag -1) kept in
// their own document by a boolean mask; constructor parameters -- 56 heads of
// 128 channels.  Computes, per head, O_i = sum_j softmax_j(scale q_i.k_j) v_j
// over the keys j of row i's document (scale 1/sqrt(128) by default).
//
// Design (one workgroup = one head x one tile of BM query rows):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16.  The A operand is a 32-key slab
//    of K read from LDS, the B operand Q^T lives in registers for the whole
//    loop.  In the accumulator every lane then holds ONE query row (lane % 32)
//    and 16 keys, so the row max / row sum need one cross-half exchange
//    (v_permlane32_swap) and the O rescale is a per-lane scalar.
//  * The K slab is read through a row permutation chosen so that accumulator
//    register 8c+t of lane half h is key 16c + 8h + t: the same registers,
//    converted to bf16, are the B operand P^T of O^T = V^T P^T with no data
//    movement, and V^T (pre-transposed by the prep kernel, keys contiguous)
//    is read from LDS in natural key order as the A operand.
//  * Online softmax in fp32 with exp2 (log2 e folded into the scale), row sum
//    by v_dot2 on the bf16 probabilities actually fed to the PV product, and
//    the O rescale skipped when no row max grew.
//  * Tiles come from the layout's per-q-tile list of non-EMPTY k-tiles: EMPTY
//    tiles are never visited; FULL tiles take no mask ops; PARTIAL tiles and
//    the ragged last k-tile mask by document bit / bounds from two ballots.
//  * K and V^T tiles are double-buffered in LDS and filled by direct-to-LDS
//    loads (global_load_lds_dwordx4): the next listed tile streams into the
//    idle buffer while the current one is consumed, with no staging
//    registers; one wait + barrier per tile.  Each wave-instruction fills
//    1 KB of LDS in lane order, so instead of row padding the 16-byte chunks
//    of a row are XOR-swizzled (chosen by the global address each lane
//    fetches), which keeps the MFMA-operand reads bank-conflict-free.
//  * Launch order is XCD-aware: the dispatcher deals workgroups round-robin
//    to the 8 XCDs, so workgroup b runs item (b % 8) * per_xcd + b / 8 and
//    each XCD sweeps whole heads, keeping that head's K/V in its own L2.
//    Within a head, q-tiles run heaviest first (the layout's order list).
#include "internal.h"

#include <cmath>

namespace pma {
namespace {

constexpr int kBN = 64;                    // keys per tile
constexpr int kD = kHeadDim;               // 128
constexpr int kTileElems = kBN * kD;       // 8192 bf16 = 16 KB per K or V^T tile

// LDS placement of 16-byte chunk c of a tile row:
//   K tile   [64 keys][16 chunks]: position c ^ (row & 15)
//   V^T tile [128 channels][8 chunks]: position c ^ ((row >> 1) & 7)
__device__ __forceinline__ int k_pos(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int v_pos(int row, int c) { return c ^ ((row >> 1) & 7); }

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS (lane l lands at
// lds + 16*l).  Kept out of the kernel template: with the builtin written in
// the template body the host compilation pass drops the kernel's stub.
__device__ __forceinline__ void dma16(const void *g, lds_void *l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// Row of the 32-key K slab that lane i supplies as MFMA A-operand row i.
// The 32x32 accumulator row of register v in lane half h is
// i = 8*(v/4) + 4*h + v%4; reading key rho(i) there makes register v hold
// key 16*(v/8) + 8*h + v%8.
__device__ __forceinline__ int k_slab_row(int i) {
    const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
    return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

// Combine a value with the same lane of the other 32-lane half.  The swap
// leaves {own value, partner value} in the two results of every lane.
__device__ __forceinline__ float half_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int NW, int QB>
__global__ __launch_bounds__(NW * 64, 2) void flash_fwd_kernel(FlashLaunch a) {
    constexpr int BM = NW * 32 * QB;
    constexpr int KI = 16 / NW;   // 1 KB direct-to-LDS instructions per wave for K (and for V^T)
    static_assert(KI * NW == 16, "16 KB tiles split over the waves");

    // two buffers per operand as four distinct objects, so the compiler can
    // tell the buffer being streamed into from the one being read
    __shared__ __attribute__((aligned(1024))) uint16_t ks0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t ks1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t vs0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t vs1[kTileElems];
    // this q-tile's k-tile list, entry = kt | (needs_mask << 30); dynamic LDS
    // of 4 * num_k_tiles bytes.  Reading it from LDS inside the loop keeps the
    // loop free of vector-memory loads that would wait on the tile stream.
    extern __shared__ int32_t tlist[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // ---- work item (XCD-aware)
    const int total = a.H * a.nqt;
    const int per_xcd = (total + 7) / 8;
    const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (item >= total) return;
    const int head = item / a.nqt;
    const int qt = a.order[item % a.nqt];
    const int cnt = a.count[qt];
    const int32_t *list = a.list + (int64_t)qt * a.nkt;
    const uint8_t *cls = a.cls + (int64_t)qt * a.nkt;
    const uint16_t *kbase = a.kh + (int64_t)head * a.Lp * kD;
    const uint16_t *vbase = a.vt + (int64_t)head * kD * a.Lp;

    // ---- Q^T fragments: lane holds query row l32, channels 16c + 8*hi + [0, 8)
    const int q0 = qt * BM + wave * 32 * QB;
    bf16x8 qf[QB][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const uint16_t *qrow = a.qh + ((int64_t)head * a.Lp + q0 + qb * 32 + l32) * kD + 8 * hi;
#pragma unroll
        for (int c = 0; c < 8; ++c) qf[qb][c] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * c);
    }

    // ---- direct-to-LDS tile loads.  Wave-instruction j of the K tile fills
    // rows 4j..4j+3 (lane l: row 4j + l/16, position l%16); of the V^T tile,
    // rows 8j..8j+7 (lane l: row 8j + l/8, position l%8).  Each lane fetches
    // the chunk the swizzle places at its position.
    // byte offsets, 32-bit, so each load is SGPR base + VGPR offset
    uint32_t kg[KI], vg[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int j = wave * KI + i;
        const int kr = 4 * j + (lane >> 4), kp = lane & 15;
        kg[i] = 2u * (uint32_t)(kr * kD + 8 * k_pos(kr, kp));
        const int vr = 8 * j + (lane >> 3), vp = lane & 7;
        vg[i] = 2u * ((uint32_t)vr * (uint32_t)a.Lp + 8u * v_pos(vr, vp));
    }
#define PMA_DMA_TILE(kt_, kdst_, vdst_)                                                      \
    do {                                                                                     \
        const char *kgb_ = reinterpret_cast<const char *>(kbase + (int64_t)(kt_) * kBN * kD); \
        const char *vgb_ = reinterpret_cast<const char *>(vbase + (int64_t)(kt_) * kBN);    \
        _Pragma("unroll") for (int i = 0; i < KI; ++i) {                                     \
            const int j = wave * KI + i;                                                     \
            dma16(kgb_ + kg[i], (lds_void *)&(kdst_)[j * 512]);                              \
            dma16(vgb_ + vg[i], (lds_void *)&(vdst_)[j * 512]);                              \
        }                                                                                    \
    } while (0)

    // ---- per-row state
    float m[QB], lsum[QB];
    int dq[QB];
    f32x16 o[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        lsum[qb] = 0.f;
        const int qrow = q0 + qb * 32 + l32;
        dq[qb] = qrow < a.L ? a.doc[qrow] : 0;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[qb][db][v] = 0.f;
    }
    const float c2 = a.scale_log2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    const int krow = k_slab_row(l32);

    for (int i = tid; i < cnt; i += NW * 64) {
        const int kt = list[i];
        const bool m = cls[kt] != PMA_TILE_FULL || (kt + 1) * kBN > a.L;
        tlist[i] = kt | (m ? (1 << 30) : 0);
    }
    PMA_DMA_TILE(list[0], ks0, vs0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    auto step = [&](int it, const uint16_t *ksr, const uint16_t *vsr, uint16_t *ksw,
                    uint16_t *vsw) __attribute__((always_inline)) {
        const int entry = tlist[it];
        const int kt = entry & 0x3fffffff;
        // stream the next listed tile into the idle buffers
        if (it + 1 < cnt) PMA_DMA_TILE(tlist[it + 1] & 0x3fffffff, ksw, vsw);

        // ---- S^T = K Q^T for two 32-key slabs
        f32x16 s[QB][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int v = 0; v < 16; ++v) s[qb][kb][v] = 0.f;
            const int r = 32 * kb + krow;
            const uint16_t *kp = ksr + r * kD;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kp + 8 * k_pos(r, 2 * c + hi));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][c], s[qb][kb],
                                                                        0, 0, 0);
            }
        }

        // ---- mask (PARTIAL tiles and the ragged tail only)
        if (entry >> 30) {
            const int key = kt * kBN + lane;
            const int dk = key < a.L ? a.doc[key] : -1;
            const uint64_t padm = __ballot(dk == 1), realm = __ballot(dk == 0);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const uint64_t allow = dq[qb] ? padm : realm;
                // the lane's 32 keys are the bytes 16g + 8*hi (g = 0..3) of the
                // tile; gather them so bit 16*kb + v is register (kb, v)
                const uint32_t lo = (uint32_t)allow, hi32 = (uint32_t)(allow >> 32);
                const uint32_t sh = 8u * hi;
                const uint32_t m32 = ((lo >> sh) & 0xffu) | (((lo >> (16 + sh)) & 0xffu) << 8) |
                                     (((hi32 >> sh) & 0xffu) << 16) |
                                     (((hi32 >> (16 + sh)) & 0xffu) << 24);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (!((m32 >> (16 * kb + v)) & 1u)) s[qb][kb][v] = -INFINITY;
            }
        }
        // ---- online softmax; P^T in bf16 straight from the accumulator registers
        bf16x8 pf[QB][4];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = s[qb][0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[qb][kb][v]);
            mx = half_max(mx);
            const float m_new = fmaxf(m[qb], mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f((m[qb] - m_use) * c2);
            const bool grow = m_new > m[qb];
            m[qb] = m_new;
            const float mc = m_use * c2;
            float rs = 0.f;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                bf16x2 pp[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][cc >> 1][8 * (cc & 1) + 2 * t], c2, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][cc >> 1][8 * (cc & 1) + 2 * t + 1], c2, -mc));
                    const f32x2 pv = {p0, p1};
                    pp[t] = __builtin_convertvector(pv, bf16x2);
                    rs = __builtin_amdgcn_fdot2_f32_bf16(pp[t], ones, rs, false);
                }
                pf[qb][cc] = __builtin_shufflevector(
                    __builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                    __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
            }
            lsum[qb] = fmaf(lsum[qb], alpha, rs);
            if (__ballot(grow)) {
#pragma unroll
                for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
            }
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int d = 32 * db + l32;
            const uint16_t *vp = vsr + d * kBN;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(vp + 8 * v_pos(d, 2 * cc + hi));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][cc], o[qb][db],
                                                                        0, 0, 0);
            }
        }

        __builtin_amdgcn_s_waitcnt(0);   // the streamed tile has landed
        __syncthreads();
    };

    for (int it = 0; it < cnt; it += 2) {
        step(it, ks0, vs0, ks1, vs1);
        if (it + 1 < cnt) step(it + 1, ks1, vs1, ks0, vs0);
    }

    // ---- epilogue: O row = O^T column / row sum; register v of d-block db is
    // channel 32*db + 8*(v/4) + 4*hi + v%4
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = half_sum(lsum[qb]);
        const float inv = 1.0f / lt;
        const int qrow = q0 + qb * 32 + l32;
        if (qrow < a.L) {
            uint16_t *orow = a.o + (int64_t)qrow * a.o_ld + head * kD + 4 * hi;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint2 w;
                    w.x = pack_bf16x2(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv);
                    w.y = pack_bf16x2(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
                    *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * g) = w;
                }
            if (a.lse && hi == 0) a.lse[(int64_t)head * a.L + qrow] = m[qb] * a.scale + logf(lt);
        }
    }
}

#undef PMA_DMA_TILE

// The instance used: 4 waves x 32 rows per wave -> 128-row q-tiles, 64-key k-tiles.
constexpr int kNW = 4, kQB = 1;

}  // namespace

void flash_tiles(int32_t *tile_m, int32_t *tile_n) {
    *tile_m = kNW * 32 * kQB;
    *tile_n = kBN;
}

hipError_t launch_flash_attention(const FlashLaunch &a, hipStream_t s) {
    const int total = a.H * a.nqt;
    const int per_xcd = (total + 7) / 8;
    flash_fwd_kernel<kNW, kQB><<<8 * per_xcd, kNW * 64, 4 * a.nkt, s>>>(a);
    return hipGetLastError();
}

}  // namespace pma
