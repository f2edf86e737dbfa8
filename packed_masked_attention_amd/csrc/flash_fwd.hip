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
//  * Online softmax in fp32 with exp2 (log2 e folded into the scale) and a
//    lazy reference max: a row's reference only moves when its max grows by
//    more than 2^8 (so p <= 256, exact in fp32/bf16 range), which makes the
//    O rescale rare.  Row sums by v_dot2 on the bf16 probabilities actually
//    fed to the PV product.
//  * Software pipelined: iteration j issues S(j+1) = K(j+1) Q^T in the same
//    basic block as the softmax of S(j), so the MFMAs of one overlap the VALU
//    of the other inside a wave; then O += V(j)^T P(j).  The K and V buffers
//    run one tile apart (K(j+1) and V(j) are resident during iteration j).
//  * Tiles come from the layout's per-q-tile list of non-EMPTY k-tiles: EMPTY
//    tiles are never visited; FULL tiles take no mask ops; PARTIAL tiles and
//    the ragged last k-tile mask by document bit / bounds from two ballots.
//  * K and V^T tiles are double-buffered in LDS and filled by direct-to-LDS
//    buffer loads (buffer_load_dwordx4 ... lds) with the tile offset in an
//    SGPR: the next tiles stream into the idle buffers while the current ones
//    are consumed, with no staging registers and no per-tile address VALU;
//    one wait + barrier per tile.  Each wave-instruction fills
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

// Buffer resource word 3 for raw (untyped) dword loads.
constexpr int kRsrcFlags = 0x00020000;

// 16 bytes per lane from a buffer straight into LDS: lane l reads
// base + voff + soff and lands at lds + 16*l.  Kept out of the kernel
// template: with the builtin written in the template body the host
// compilation pass drops the kernel's stub.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_void *l, uint32_t voff,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcFlags);
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

template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void flash_fwd_kernel(FlashLaunch a) {
    constexpr int BM = NW * 32;
    constexpr int KI = 16 / NW;   // 1 KB LDS-DMA instructions per wave per tile (K or V^T)
    static_assert(KI * NW == 16, "16 KB tiles split over the waves");
    constexpr int kMask = 0x3fffffff;

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
    {
        const int32_t *list = a.list + (int64_t)qt * a.nkt;
        const uint8_t *cls = a.cls + (int64_t)qt * a.nkt;
        for (int i = tid; i < cnt; i += NW * 64) {
            const int kt = list[i];
            const bool m = cls[kt] != PMA_TILE_FULL || (kt + 1) * kBN > a.L;
            tlist[i] = kt | (m ? (1 << 30) : 0);
        }
    }
    __syncthreads();   // the list is read by every wave from here on
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(a.kh + (int64_t)head * a.Lp * kD, (uint32_t)a.Lp * kD * 2u);
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(a.vt + (int64_t)head * kD * a.Lp, (uint32_t)a.Lp * kD * 2u);

    // ---- Q^T fragments: lane holds query row l32, channels 16c + 8*hi + [0, 8)
    const int q0 = qt * BM + wave * 32;
    bf16x8 qf[8];
    {
        const uint16_t *qrow = a.qh + ((int64_t)head * a.Lp + q0 + l32) * kD + 8 * hi;
#pragma unroll
        for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * c);
    }

    // ---- LDS-DMA lane offsets.  Wave-instruction j of the K tile fills rows
    // 4j..4j+3 (lane l: row 4j + l/16, position l%16); of the V^T tile, rows
    // 8j..8j+7 (lane l: row 8j + l/8, position l%8).  Each lane fetches the
    // chunk the swizzle places at its position; the tile's own offset
    // (kt * 64 keys) is the SGPR offset.
    uint32_t kvo[KI], vvo[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int j = wave * KI + i;
        const int kr = 4 * j + (lane >> 4), kp = lane & 15;
        kvo[i] = 2u * (uint32_t)(kr * kD + 8 * k_pos(kr, kp));
        const int vr = 8 * j + (lane >> 3), vp = lane & 7;
        vvo[i] = 2u * ((uint32_t)vr * (uint32_t)a.Lp + 8u * v_pos(vr, vp));
    }
    auto dma_k = [&](int kt, uint16_t *dst) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KI; ++i)
            dma16(krs, (lds_void *)&dst[(wave * KI + i) * 512], kvo[i], (uint32_t)kt * (kBN * kD * 2));
    };
    auto dma_v = [&](int kt, uint16_t *dst) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KI; ++i)
            dma16(vrs, (lds_void *)&dst[(wave * KI + i) * 512], vvo[i], (uint32_t)kt * (kBN * 2));
    };

    // ---- S^T = K Q^T over one K tile: two 32-key slabs
    const int krow = k_slab_row(l32);
    auto qk = [&](const uint16_t *kbuf, f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
            const int r = 32 * kb + krow;
            const uint16_t *kp = kbuf + r * kD;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kp + 8 * k_pos(r, 2 * c + hi));
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
            }
        }
    };

    // ---- document / bounds mask of a PARTIAL or ragged tile
    const int qrow = q0 + l32;
    const int dq = (uint32_t)qrow < (uint32_t)a.L ? a.doc[qrow] : 0;
    auto apply_mask = [&](int kt, f32x16 (&s)[2]) __attribute__((always_inline)) {
        const int key = kt * kBN + lane;
        const int dk = (uint32_t)key < (uint32_t)a.L ? a.doc[key] : -1;
        const uint64_t padm = __ballot(dk == 1), realm = __ballot(dk == 0);
        const uint64_t allow = dq ? padm : realm;
        // the lane's 32 keys are the bytes 16g + 8*hi (g = 0..3) of the tile;
        // gather them so bit 16*kb + v is register (kb, v)
        const uint32_t lo = (uint32_t)allow, hw = (uint32_t)(allow >> 32);
        const uint32_t sh = 8u * hi;
        const uint32_t m32 = ((lo >> sh) & 0xffu) | (((lo >> (16 + sh)) & 0xffu) << 8) |
                             (((hw >> sh) & 0xffu) << 16) | (((hw >> (16 + sh)) & 0xffu) << 24);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (!((m32 >> (16 * kb + v)) & 1u)) s[kb][v] = -INFINITY;
    };

    // ---- per-row state: lazy reference max (log2 units), partial row sum, O^T
    float mref = -INFINITY, lsum = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
    const float c2 = a.scale_log2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // ---- prologue: K(0), V(0), K(1) resident; S(0) computed and masked
    f32x16 s[2];
    {
        const int e0 = tlist[0];
        dma_k(e0 & kMask, ks0);
        dma_v(e0 & kMask, vs0);
        if (cnt > 1) dma_k(tlist[1] & kMask, ks1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        qk(ks0, s);
        if (e0 >> 30) apply_mask(e0 & kMask, s);
        __syncthreads();   // every wave is done with ks0 before it is refilled
    }

    // iteration j: reads K(j+1) from kr and V(j) from vr; streams K(j+2) into
    // kw and V(j+1) into vw
    auto step = [&](int j, const uint16_t *kr, uint16_t *kw, const uint16_t *vr, uint16_t *vw)
                    __attribute__((always_inline)) {
        const bool has1 = j + 1 < cnt;
        const int e1 = has1 ? tlist[j + 1] : 0;
        if (j + 2 < cnt) dma_k(tlist[j + 2] & kMask, kw);
        if (has1) dma_v(e1 & kMask, vw);

        // S(j+1): issued unconditionally (a stale buffer past the end is read
        // and discarded) so it shares a basic block with the softmax below
        f32x16 sn[2];
        qk(kr, sn);

        // softmax of S(j) -> P(j)^T in bf16
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
        mx = half_max(mx) * c2;
        const bool need = mx > mref + 8.0f;
        const float mnew = need ? mx : mref;
        const float alpha = need ? __builtin_amdgcn_exp2f(mref - mnew) : 1.0f;
        mref = mnew;
        const float mu = (mnew == -INFINITY) ? 0.f : mnew;
        float rs = 0.f;
        bf16x8 pf[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            bf16x2 pp[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[cc >> 1][8 * (cc & 1) + 2 * t], c2, -mu));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[cc >> 1][8 * (cc & 1) + 2 * t + 1], c2, -mu));
                const f32x2 pv = {p0, p1};
                pp[t] = __builtin_convertvector(pv, bf16x2);
                rs = __builtin_amdgcn_fdot2_f32_bf16(pp[t], ones, rs, false);
            }
            pf[cc] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                             __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                             0, 1, 2, 3, 4, 5, 6, 7);
        }
        lsum = fmaf(lsum, alpha, rs);
        // interleave S(j+1)'s MFMAs with the softmax VALU: K fragment reads run
        // two ahead, then 16 x {1 MFMA, 1 LDS read, 6 VALU}
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
        // the row sum in the condition (never negative) keeps the softmax
        // above this branch, in the block it shares with S(j+1)'s MFMAs
        if (__ballot(need || !(rs >= 0.f))) {
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] *= alpha;
        }

        // O^T += V(j)^T P(j)^T
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int d = 32 * db + l32;
            const uint16_t *vp = vr + d * kBN;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(vp + 8 * v_pos(d, 2 * cc + hi));
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[cc], o[db], 0, 0, 0);
            }
        }

        if (has1 && (e1 >> 30)) apply_mask(e1 & kMask, sn);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = sn[kb];
        __builtin_amdgcn_s_waitcnt(0);   // the streamed tiles have landed
        __syncthreads();
    };

    for (int j = 0; j < cnt; j += 2) {
        step(j, ks1, ks0, vs0, vs1);
        if (j + 1 < cnt) step(j + 1, ks0, ks1, vs1, vs0);
    }

    // ---- epilogue: O row = O^T column / row sum; register v of d-block db is
    // channel 32*db + 8*(v/4) + 4*hi + v%4
    const float lt = half_sum(lsum);
    const float inv = 1.0f / lt;
    if (qrow < a.L) {
        uint16_t *orow = a.o + (int64_t)qrow * a.o_ld + head * kD + 4 * hi;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 w;
                w.x = pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
                w.y = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * g) = w;
            }
        if (a.lse && hi == 0)
            a.lse[(int64_t)head * a.L + qrow] = (mref + __log2f(lt)) * 0.69314718055994531f;
    }
}

// The instance used: 4 waves x 32 query rows -> 128-row q-tiles, 64-key k-tiles.
constexpr int kNW = 4;

}  // namespace

void flash_tiles(int32_t *tile_m, int32_t *tile_n) {
    *tile_m = kNW * 32;
    *tile_n = kBN;
}

hipError_t launch_flash_attention(const FlashLaunch &a, hipStream_t s) {
    const int total = a.H * a.nqt;
    const int per_xcd = (total + 7) / 8;
    flash_fwd_kernel<kNW><<<8 * per_xcd, kNW * 64, 4 * a.nkt, s>>>(a);
    return hipGetLastError();
}

}  // namespace pma
