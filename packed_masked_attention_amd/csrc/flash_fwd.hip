// flash_fwd.hip -- masked flash attention forward for gfx950 (bf16 MFMA).
//
// Page "MiniMaxH3Transformer3DModel" (diffusers API page): intro -- full
// self-attention over the packed sequence, padding rows (tag -1) kept in
// their own document by a boolean mask; constructor parameters -- 56 heads of
// 128 channels.  Computes, per head, O_i = sum_j softmax_j(scale q_i.k_j) v_j
// over the keys j of row i's document (scale 1/sqrt(128) by default).
//
// Design (one workgroup = one head x one tile of 256 query rows, 8 waves):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16.  The A operand is a 32-key slab
//    of K read from LDS, the B operand Q^T lives in registers for the whole
//    loop.  In the accumulator every lane then holds ONE query row (lane % 32)
//    and half of the tile's keys, so the row max / row sum need one
//    cross-half exchange (v_permlane32_swap) and the O rescale is a per-lane
//    scalar.
//  * The K slab is read through a row permutation chosen so that accumulator
//    register 8c+t of lane half h is key 16c + 8h + t: the same registers,
//    converted to bf16, are the B operand P^T of O^T = V^T P^T with no data
//    movement, and V^T (pre-transposed by the prep kernel, keys contiguous)
//    is read from LDS in natural key order as the A operand.
//  * Ping-pong between two wave groups.  Waves w and w+4 share a SIMD; group
//    0 (waves 0-3) and group 1 (waves 4-7) alternate, one barrier-separated
//    phase apart, between an MFMA phase G(t) = {O += V(t-1)^T P(t-1)^T,
//    S(t) = K(t) Q^T} (32 MFMAs, raised wave priority) and a softmax phase
//    S(t) (VALU only).  While one wave of a SIMD runs its MFMAs the other runs
//    its softmax, so matrix and vector units work at the same time; within a
//    phase nothing waits on the other unit.
//  * Softmax in fp32 with exp2.  Q' carries the logit scale (softmax_scale *
//    log2 e, applied where Q' is produced), and the QK accumulators of a row
//    start from minus its reference instead of zero, so the MFMA delivers
//    log2-unit logits relative to the reference and p = exp2(s) needs no
//    per-score arithmetic.  The reference is lazy: it only moves when the
//    row's max grows by more than 2^8 (so p <= 256), which makes the O
//    rescale rare (it then also shifts that tile's scores).  Each half of a
//    row first tests its own keys against that threshold; the exchange of
//    the halves' maxima and the rescale run only in a wave where some row
//    crossed it (a wave-uniform branch, taken on the first tiles of a work
//    item and rarely after).  The row max is four independent chains of three-input IEEE maximum (NaN-propagating,
//    so the raw MFMA results need no canonicalising first) and the row sum
//    four independent add chains: the softmax wave has no other wave to hide
//    its latencies behind.
//  * K, V^T tiles (64 keys) stream through a 4-deep LDS ring filled by
//    direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds) with the tile
//    offset in an SGPR.  Every wave issues its share of tile t+3's K and
//    t+2's V^T at the start of its softmax phase S(t), so the MFMA phase's
//    issue slots stay with the MFMAs and their fragment reads (issued inside
//    the MFMA phase, even spread one every few MFMAs, they cost 2-8%); every
//    phase end waits for all but the newest batch, so a batch lands within
//    S(t), G(t+1) and S(t+1) and no wave waits for a tile it just requested.
//    The 64 document ids of a V tile's keys ride along in the same slot (for
//    the rare masked tile).
//    Each 1 KB wave-instruction fills LDS in lane order, so instead of row
//    padding the 16-byte chunks of a row are XOR-swizzled (chosen by the
//    global address each lane fetches), which keeps the MFMA-operand reads
//    bank-conflict-free.
//  * Tiles come from the layout's per-q-tile list of non-EMPTY k-tiles, copied
//    to LDS (entry = kt | needs_mask << 30): EMPTY tiles are never visited,
//    FULL tiles take no mask ops, PARTIAL and ragged tiles mask by document /
//    bounds with two ballots.
//  * Launch order is XCD-aware: the dispatcher deals workgroups round-robin
//    to the 8 XCDs, so workgroup b runs item (b % 8) * per_xcd + b / 8 and
//    each XCD sweeps whole heads, keeping that head's K/V in its own L2.
//    Within a head, q-tiles run heaviest first (the layout's order list).
//  * Load balance (with a work-queue buffer): one workgroup per CU stays
//    resident and pulls work units from atomic counters -- its own XCD's
//    items first, then what is left of the other XCDs' shares.  The hardware
//    deals workgroups to the XCDs, and within an XCD to its shader engines,
//    in a fixed round-robin order, so with one item per workgroup a CU can
//    wait for its turn while items of unequal cost (a masked layout's light
//    padding q-tiles) and XCDs of unequal speed (on MI355X up to 10% apart
//    on the same items) leave others idle.  The last units are parts: the
//    last kSplitItems items of every XCD's share, each split over
//    consecutive halves (below 12288 keys) or quarters of its key list, so
//    the final units are short.  A
//    part writes its unnormalised O, reference max and row sum, and
//    flash_merge_kernel combines the parts (the split form of the online
//    softmax: weights 2^(m_p - m) on each part's O and row sum).
#include "internal.h"

#include <cmath>

namespace pma {
namespace {

constexpr int kNW = 8;                     // waves per workgroup
constexpr int kBM = kNW * 32;              // 256 query rows per workgroup
constexpr int kBN = 64;                    // keys per tile
constexpr int kD = kHeadDim;               // 128
constexpr int kTileElems = kBN * kD;       // 8192 bf16 = 16 KB per K or V^T tile
constexpr int kKI = 16 / kNW;              // 1 KB LDS-DMA instructions per wave per tile
constexpr int kNDMA = 2 * kKI + 1;         // DMA instructions per wave per tile (K, V^T, ids)
constexpr int kReadAhead = 3;              // LDS fragment reads in flight ahead of the MFMAs
constexpr int kVPre = 2;                   // V fragments read during the softmax phase
constexpr int kMask = 0x3fffffff;          // list entry -> k-tile index
constexpr int kSplitItems = 16;            // items per XCD split over their key range
constexpr int kSplitMinKeyTiles = 128;     // no work queue below this many k-tiles (8192 keys)
constexpr int kMaxSplitParts = 4;          // partial-result slots per split item
constexpr int kFourPartMinKeyTiles = 192;  // 4 parts per split item from here (12288 keys), 2 below
// one part's partial result: O [kBM rows][kD] fp32, then (m, l) per row
constexpr int kPartFloats = kBM * kD + 2 * kBM;
static_assert(kFlashQueueBytes >= 16 * sizeof(int32_t), "the queue reset clears 16 counters");
// LDS: 4 K slots + 4 V^T slots (each + 64 document ids) + the tile list
// (the V^T slots are 1024-byte aligned, so each takes 17 KB; 1 KB more covers
// the work-item word and any placement slack of the static variables)
constexpr int kStaticLds = 4 * kTileElems * 2 + 4 * (((kTileElems + 2 * kBN) * 2 + 1023) / 1024 * 1024) + 1024;
constexpr int kLdsBytes = 160 * 1024;      // per workgroup on gfx950
static_assert(kKI * kNW == 16, "16 KB tiles split over the waves");

// LDS placement of 16-byte chunk c of a tile row:
//   K tile   [64 keys][16 chunks]: position c ^ (row & 15)
//   V^T tile [128 channels][8 chunks]: position c ^ ((row >> 1) & 7)
__device__ __forceinline__ int k_pos(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int v_pos(int row, int c) { return c ^ ((row >> 1) & 7); }

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource word 3 for raw (untyped) dword loads.
constexpr int kRsrcFlags = 0x00020000;

// 16 (or 4) bytes per lane from a buffer straight into LDS: lane l reads
// base + voff + soff and lands at lds + 16*l (4*l); reads past the
// resource's size return 0.  Kept out of the kernel template: with the
// builtin written in the template body the host compilation pass drops the
// kernel's stub.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_void *l, uint32_t voff,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, lds_void *l, uint32_t voff,
                                     uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 4, voff, soff, 0, 0);
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
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
#define PMA_WAIT_VM(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
// End of a phase: this wave's LDS reads done and all but its newest n DMA
// instructions landed, then the workgroup barrier -- a plain s_barrier (asm
// with a memory clobber, so no memory access moves across it): the release
// fence of __syncthreads() would wait for every DMA in flight.
#define PMA_PHASE_END(n)                                                                   \
    do {                                                                                    \
        __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (((n) >> 4) << 14));           \
        asm volatile("s_barrier" ::: "memory");                                            \
    } while (0)

// The next unit of work of a workgroup: {item, part} (part -1: the whole
// item; item -1: none left).  Without a work queue workgroup b takes item
// (b % 8) * per_xcd + b / 8 and nothing more: the dispatcher deals
// workgroups round-robin to the 8 XCDs, so each XCD sweeps whole heads.  With
// one, the workgroups persist (one per CU) and pull units until none is left:
// first the items of their own XCD's share (local indices [0, per_xcd - S),
// in order, so its heads' K/V stay in its L2), then the remaining items of
// the other XCDs' shares (neighbours first), then the split_parts parts of
// the last S items of every share: its own XCD's parts first (their heads'
// K/V sit in its L2), then the others' (neighbours first).  An XCD that runs
// ahead takes over the tail of a slower one's share.
// Workgroups per split item: 2 below 12288 keys, 4 from there (at 8192 keys,
// 1.4513 ms with 2 parts, 1.4724 with 4, 1.4743 without the queue; at 16384
// keys 2 or 8 parts were 0.5-0.7% slower than 4).
__device__ __forceinline__ int split_parts(const FlashLaunch &a) {
    return a.nkt < kFourPartMinKeyTiles ? 2 : kMaxSplitParts;
}

__device__ __forceinline__ int2 next_work(const FlashLaunch &a, int xcd, int iter) {
    const int total = a.H * a.nqt;
    const int per_xcd = (total + 7) / 8;
    if (!a.queue) {
        const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
        return make_int2(iter == 0 && item < total ? item : -1, -1);
    }
    const int S = a.split_items, P = split_parts(a);
    for (int k = 0; k < 8; ++k) {
        const int y = (xcd + k) & 7;
        const int own = min(per_xcd - S, max(0, total - y * per_xcd));
        // skip a share that is already handed out without touching its counter
        if (k > 0 && __hip_atomic_load(&a.queue[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= own)
            continue;
        const int w = atomicAdd(&a.queue[y], 1);
        if (w < own) return make_int2(y * per_xcd + w, -1);
    }
    // parts: this XCD's own first (its heads' K/V are in its L2), then the
    // other XCDs' (neighbours first)
    for (int k = 0; k < 8; ++k) {
        const int y = (xcd + k) & 7;
        if (__hip_atomic_load(&a.queue[8 + y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= S * P)
            continue;
        for (;;) {
            const int g = atomicAdd(&a.queue[8 + y], 1);
            if (g >= S * P) break;
            const int item = y * per_xcd + per_xcd - S + g / P;
            if (item < total) return make_int2(item, g % P);
        }
    }
    return make_int2(-1, -1);
}

typedef __attribute__((address_space(4))) const FlashLaunch *kernarg_launch;

__global__ __launch_bounds__(kNW * 64, 1) void flash_fwd_kernel(FlashLaunch arg) {
    // ring slots as distinct objects, so the compiler can tell the slot being
    // streamed into from the ones being read
    __shared__ __attribute__((aligned(1024))) uint16_t ks0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t ks1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t ks2[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t ks3[kTileElems];
    // V^T tile, then the document ids of its 64 keys (int32)
    __shared__ __attribute__((aligned(1024))) uint16_t vs0[kTileElems + 2 * kBN];
    __shared__ __attribute__((aligned(1024))) uint16_t vs1[kTileElems + 2 * kBN];
    __shared__ __attribute__((aligned(1024))) uint16_t vs2[kTileElems + 2 * kBN];
    __shared__ __attribute__((aligned(1024))) uint16_t vs3[kTileElems + 2 * kBN];
    // this q-tile's k-tile list, entry = kt | (needs_mask << 30), then 4 pad
    // entries (tile 0) for the lookahead past the end: dynamic LDS of
    // 4 * (num_k_tiles + 4) bytes.  Reading it from LDS inside the loop keeps
    // the loop free of vector-memory loads that would wait on the tile stream.
    extern __shared__ int32_t tlist[];

    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform by construction; readfirstlane keeps everything derived from
    // it (LDS-DMA destinations, row offsets) on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int l32 = lane & 31, hi = lane >> 5;

    // the XCD this workgroup runs on (hardware register XCC_ID)
    const int xcd_hw = (int)(__builtin_amdgcn_s_getreg(20 | (15 << 11)) & 7);
    __shared__ int2 work;
    (void)arg;   // read through the kernarg segment below
    if (tid == 0) {
        // clock stamps (persistent launches with a workspace): shader clock
        // and 100 MHz real-time clock at the workgroup's start
        uint64_t *st = ((kernarg_launch)__builtin_amdgcn_kernarg_segment_ptr())->stamps;
        if (st) {
            st[4 * blockIdx.x] = __builtin_amdgcn_s_memtime();
            st[4 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
        }
    }
    for (int iter = 0;; ++iter) {
        // the launch arguments, read again for every item, so that none of them
        // stays live across the work loop
        kernarg_launch ap = (kernarg_launch)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        FlashLaunch a;
        __builtin_memcpy(&a, ap, sizeof(FlashLaunch));
        if (tid == 0) work = next_work(a, xcd_hw, iter);
        __syncthreads();
        const int item = __builtin_amdgcn_readfirstlane(work.x);
        const int part = __builtin_amdgcn_readfirstlane(work.y);
        __syncthreads();   // every wave has read `work` before it is written again
        if (item < 0) break;
        const int total = a.H * a.nqt;
        const int per_xcd = (total + 7) / 8;
        const int head = item / a.nqt;
        const int qt = a.order[item % a.nqt];
        const int full = a.count[qt];
        const int nparts = split_parts(a);
        const int beg = part < 0 ? 0 : part * full / nparts;
        const int cnt = part < 0 ? full : (part + 1) * full / nparts - beg;
        // a part's partial result: slot of (owning XCD, split item, part)
        const int owner = item / per_xcd, sidx = item % per_xcd - (per_xcd - a.split_items);
        float *pres = part < 0 ? nullptr
                               : a.part + (int64_t)((owner * a.split_items + sidx) * kMaxSplitParts + part) *
                                              kPartFloats;
        if (cnt == 0) {
            // an empty key range: a part with no weight
            if (tid < kBM) {
                pres[kBM * kD + 2 * tid] = -INFINITY;
                pres[kBM * kD + 2 * tid + 1] = 0.f;
            }
            continue;
        }
        // ---- Q^T fragments: lane holds query row l32, channels 16c + 8*hi + [0, 8)
        // (requested before the tile list is copied, so the two loads' latencies
        // overlap)
        const int q0 = qt * kBM + wave * 32;
        bf16x8 qf[8];
        {
            const uint16_t *qrow = a.qh + ((int64_t)head * a.Lp + q0 + l32) * kD + 8 * hi;
#pragma unroll
            for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * c);
        }
        const int qrow = q0 + l32;
        const int dq = (uint32_t)qrow < (uint32_t)a.L ? a.doc[qrow] : 0;

        {
            const int32_t *list = a.list + (int64_t)qt * a.nkt + beg;
            const uint8_t *cls = a.cls + (int64_t)qt * a.nkt;
            for (int i = tid; i < cnt; i += kNW * 64) {
                const int kt = list[i];
                const bool m = cls[kt] != PMA_TILE_FULL || (kt + 1) * kBN > a.L;
                tlist[i] = kt | (m ? (1 << 30) : 0);
            }
            if (tid < 4) tlist[cnt + tid] = 0;
        }
        __syncthreads();   // the list is read by every wave from here on

        const __amdgpu_buffer_rsrc_t krs =
            make_rsrc(a.kh + (int64_t)head * a.Lp * kD, (uint32_t)a.Lp * kD * 2u);
        const __amdgpu_buffer_rsrc_t vrs =
            make_rsrc(a.vt + (int64_t)head * kD * a.Lp, (uint32_t)a.Lp * kD * 2u);
        // keys past the sequence read as document 0 here; the mask adds the bound
        const __amdgpu_buffer_rsrc_t drs = make_rsrc(a.doc, (uint32_t)a.L * 4u);

        // ---- LDS-DMA lane offsets.  Wave-instruction j of the K tile fills rows
        // 4j..4j+3 (lane l: row 4j + l/16, position l%16); of the V^T tile, rows
        // 8j..8j+7 (lane l: row 8j + l/8, position l%8).  Each lane fetches the
        // chunk the swizzle places at its position; the tile's own offset
        // (kt * 64 keys) is the SGPR offset.
        uint32_t kvo[kKI], vvo[kKI];
#pragma unroll
        for (int i = 0; i < kKI; ++i) {
            const int j = wave * kKI + i;
            const int kr = 4 * j + (lane >> 4), kp = lane & 15;
            kvo[i] = 2u * (uint32_t)(kr * kD + 8 * k_pos(kr, kp));
            const int vr = 8 * j + (lane >> 3), vp = lane & 7;
            vvo[i] = 2u * ((uint32_t)vr * (uint32_t)a.Lp + 8u * v_pos(vr, vp));
        }
        const uint32_t dvo = 4u * (uint32_t)(wave * 8 + (lane & 7));
        // wave-instruction i of this wave's share of a K or V^T tile, and the
        // document ids of a V tile's keys (8 per wave: lanes 0..7)
        auto dma_k1 = [&](int kt, uint16_t *dst, int i) __attribute__((always_inline)) {
            dma16(krs, (lds_void *)&dst[(wave * kKI + i) * 512], kvo[i], (uint32_t)kt * (kBN * kD * 2));
        };
        auto dma_v1 = [&](int kt, uint16_t *dst, int i) __attribute__((always_inline)) {
            dma16(vrs, (lds_void *)&dst[(wave * kKI + i) * 512], vvo[i], (uint32_t)kt * (kBN * 2));
        };
        auto dma_id = [&](int kt, uint16_t *dst) __attribute__((always_inline)) {
            if (lane < 8) dma4(drs, (lds_void *)&dst[kTileElems + wave * 16], dvo, (uint32_t)kt * (kBN * 4));
        };
        auto dma_k = [&](int kt, uint16_t *dst) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < kKI; ++i) dma_k1(kt, dst, i);
        };
        auto dma_v = [&](int kt, uint16_t *dst) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < kKI; ++i) dma_v1(kt, dst, i);
            dma_id(kt, dst);
        };

        const int krow = k_slab_row(l32);

        // ---- per-row state (log2 units): lazy reference max (-inf until the
        // row's first key), partial row sum, O^T.  mu is the offset the QK
        // accumulators start from (-mu in every register of sd): the
        // reference once set, 0 before; thr is the score (relative to mu)
        // above which the row must move its reference: 8 once set, -inf before.
        float mref = -INFINITY, lsum = 0.f;
        float thr = -INFINITY, mu = 0.f;
        f32x16 sd;
#pragma unroll
        for (int v = 0; v < 16; ++v) sd[v] = 0.f;
        f32x16 o[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
        f32x16 s[2];     // S(t)^T, 2 slabs of 32 keys
        bf16x8 pf[4];    // P(t)^T in bf16, 4 chunks of 16 keys
        bf16x8 vpre[kVPre];

        // ---- MFMA phase: O^T += V(t-1)^T P(t-1)^T (when withpv), S(t) = K(t) Q^T - mu
        auto gphase = [&](bool withpv, const uint16_t *vr, const uint16_t *kr)
                          __attribute__((always_inline)) {
            __builtin_amdgcn_s_setprio(1);
            if (withpv) {
                // channel blocks interleaved so consecutive MFMAs are independent
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        const int d = 32 * db + l32;
                        const int f = cc * 4 + db;
                        const bf16x8 vf =
                            f < kVPre ? vpre[f < kVPre ? f : 0]
                                      : *reinterpret_cast<const bf16x8 *>(
                                            vr + d * kBN + 8 * v_pos(d, 2 * cc + hi));
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[cc], o[db], 0, 0, 0);
                    }
            }
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int r = 32 * kb + krow;
                    const bf16x8 kf =
                        *reinterpret_cast<const bf16x8 *>(kr + r * kD + 8 * k_pos(r, 2 * c + hi));
                    // the first k-step starts from the seed -mu
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], c == 0 ? sd : s[kb],
                                                                    0, 0, 0);
                }
            // LDS fragment reads run kReadAhead ahead of their MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, kReadAhead, 0);
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_s_setprio(0);
        };

        // ---- softmax phase of tile t (list entry e, V(t) slot vn): this wave's
        // share of DMA(t) = {K(t+3) into slot dks, V(t+2) into dvs}, mask,
        // lazy-max softmax -> P(t)^T in bf16, O rescale
        auto sphase = [&](int e, const uint16_t *vn, int dk, uint16_t *dks, int dv, uint16_t *dvs)
                          __attribute__((always_inline)) {
            // the ring refill first: the earlier it goes out, the longer it
            // has to land (issued after the V pre-reads or at the end of the
            // phase, 0.4% and 0.9% slower)
            dma_id(dv, dvs);
            dma_k(dk, dks);
#pragma unroll
            for (int i = 0; i < kKI; ++i) dma_v1(dv, dvs, i);
            // V(t) fragments for the first MFMAs of the next PV, read while the
            // softmax runs
#pragma unroll
            for (int f = 0; f < kVPre; ++f) {
                const int cc = f / 4, db = f % 4;
                const int d = 32 * db + l32;
                vpre[f] = *reinterpret_cast<const bf16x8 *>(vn + d * kBN + 8 * v_pos(d, 2 * cc + hi));
            }
            if (e >> 30) {
                // document / bounds mask of a PARTIAL or ragged tile.  The lane's
                // 32 keys are the bytes 16g + 8*hi (g = 0..3) of the tile's
                // ballot; gather them so bit 16*kb + v is register (kb, v)
                const int key = (e & kMask) * kBN + lane;
                const int dk = (uint32_t)key < (uint32_t)a.L
                                   ? reinterpret_cast<const int32_t *>(vn + kTileElems)[lane] : -1;
                // both ballots over the whole wave (lane = key), then the row's pick:
                // a ballot under a divergent select would drop the other lanes' keys
                const uint64_t padm = __ballot(dk == 1), realm = __ballot(dk == 0);
                const uint64_t allow = dq ? padm : realm;
                const uint32_t lo = (uint32_t)allow, hw = (uint32_t)(allow >> 32);
                const uint32_t sh = 8u * hi;
                const uint32_t m32 = ((lo >> sh) & 0xffu) | (((lo >> (16 + sh)) & 0xffu) << 8) |
                                     (((hw >> sh) & 0xffu) << 16) | (((hw >> (16 + sh)) & 0xffu) << 24);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (!((m32 >> (16 * kb + v)) & 1u)) s[kb][v] = -INFINITY;
            }
            // row max over four independent chains of IEEE maximum, which the
            // compiler fuses into three-input v_maximum3 on the raw MFMA results
            // (fmaxf would canonicalise every input first)
            float m4[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int b = 8 * (g & 1);
                float m = __builtin_elementwise_maximum(s[g >> 1][b], s[g >> 1][b + 1]);
#pragma unroll
                for (int k = 2; k < 8; k += 2)
                    m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, s[g >> 1][b + k]),
                                                      s[g >> 1][b + k + 1]);
                m4[g] = m;
            }
            float mx = __builtin_elementwise_maximum(
                __builtin_elementwise_maximum(__builtin_elementwise_maximum(m4[0], m4[1]), m4[2]), m4[3]);
            // each half tests its own 32 keys against the threshold; only a wave
            // with a row that crossed it exchanges the halves' maxima, moves
            // those rows' references, rescales their O and row sums and shifts
            // this tile's scores to the new reference
            if (__ballot(mx > thr)) {
                const float mrow = half_max(mx);           // relative to mu
                const bool need = mrow > thr;
                const float shift = need ? mrow : 0.f;
                const float mnew = need ? mu + mrow : mref;
                const float alpha = need ? __builtin_amdgcn_exp2f(mref - mnew) : 1.0f;
                mref = mnew;
                mu = need ? mnew : mu;
                thr = (mref - mu) + 8.0f;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < 4; ++db) o[db] *= alpha;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) s[kb][v] -= shift;
#pragma unroll
                for (int v = 0; v < 16; ++v) sd[v] = -mu;
            }
            // probabilities; the row sum (four independent chains, each started
            // by its first pair rather than by adding to zero) is taken over the
            // fp32 values before their rounding to bf16
            float rsp[4];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                bf16x2 pp[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float p0 = __builtin_amdgcn_exp2f(s[cc >> 1][8 * (cc & 1) + 2 * t]);
                    const float p1 = __builtin_amdgcn_exp2f(s[cc >> 1][8 * (cc & 1) + 2 * t + 1]);
                    const f32x2 pv = {p0, p1};
                    pp[t] = __builtin_convertvector(pv, bf16x2);
                    rsp[t] = cc ? rsp[t] + (p0 + p1) : p0 + p1;
                }
                pf[cc] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                                 __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
            }
            lsum += (rsp[0] + rsp[1]) + (rsp[2] + rsp[3]);
            // keep the softmax in this phase: without a use here the compiler
            // sinks it past the barrier into the MFMA phase that consumes P
            asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(pf[2]), "v"(pf[3]), "v"(lsum));
        };

        // ---- prologue: K(0..2), V(0..1) resident
        dma_k(__builtin_amdgcn_readfirstlane(tlist[0]) & kMask, ks0);
        dma_k(__builtin_amdgcn_readfirstlane(tlist[1]) & kMask, ks1);
        dma_k(__builtin_amdgcn_readfirstlane(tlist[2]) & kMask, ks2);
        dma_v(__builtin_amdgcn_readfirstlane(tlist[0]) & kMask, vs0);
        dma_v(__builtin_amdgcn_readfirstlane(tlist[1]) & kMask, vs1);
        PMA_PHASE_END(0);

        // Global phase p: group 0 runs G(t) at p = 2t and S(t) at 2t + 1; group 1
        // runs one phase later.  Tile x sits in ring slot x % 4.  K(t) is read in
        // phases 2t, 2t+1; V(t) in 2t+1 .. 2t+3.  Each wave issues its share of
        // DMA(t) = {K(t+3), V(t+2)} at the start of its S(t) (phase 2t+1 or
        // 2t+2: the slots of K(t-1) and V(t-2), both done with by the end of
        // phase 2t-1).  Every phase end leaves only the newest batch in flight,
        // so DMA(t) has landed by the end of S(t+1) (phase 2t+3 or 2t+4),
        // before V(t+2) is first read (phase 2t+5) or K(t+3) (2t+6).
        if (grp == 1) PMA_PHASE_END(0);

        // list entries of the current tile t: ce = entry t, ck = entry t+3 (the
        // K tile to fetch), cv = entry t+2 (the V tile to fetch).  The next
        // tile's are read during the softmax phase, so the MFMA phase starts
        // without an LDS wait.
        int ce = __builtin_amdgcn_readfirstlane(tlist[0]);
        int ck = __builtin_amdgcn_readfirstlane(tlist[3]);
        int cv = __builtin_amdgcn_readfirstlane(tlist[2]);
        // k_r = K(t), k_m = slot of K(t-1) <- K(t+3); v_r = V(t), v_p = V(t-1),
        // v_q = slot of V(t-2) <- V(t+2)
        auto tile = [&](int t, bool withpv, uint16_t *k_r, uint16_t *k_m, uint16_t *v_r,
                        uint16_t *v_p, uint16_t *v_q) __attribute__((always_inline)) {
            const int e = ce;
            gphase(withpv, v_p, k_r);
            PMA_PHASE_END(kNDMA);
            const int ne = tlist[t + 1], nk = tlist[t + 4], nv = tlist[t + 3];
            sphase(e, v_r, ck & kMask, k_m, cv & kMask, v_q);
            ce = __builtin_amdgcn_readfirstlane(ne);
            ck = __builtin_amdgcn_readfirstlane(nk);
            cv = __builtin_amdgcn_readfirstlane(nv);
            PMA_PHASE_END(kNDMA);
        };
        //    t, pv,   K(t) K(t-1) V(t) V(t-1) V(t-2)
        tile(0, false, ks0, ks3, vs0, vs3, vs2);
        int t = 1;
        for (; t + 4 <= cnt; t += 4) {
            tile(t, true, ks1, ks0, vs1, vs0, vs3);
            tile(t + 1, true, ks2, ks1, vs2, vs1, vs0);
            tile(t + 2, true, ks3, ks2, vs3, vs2, vs1);
            tile(t + 3, true, ks0, ks3, vs0, vs3, vs2);
        }
        // t % 4 == 1 here
        if (t < cnt) tile(t, true, ks1, ks0, vs1, vs0, vs3), ++t;
        if (t < cnt) tile(t, true, ks2, ks1, vs2, vs1, vs0), ++t;
        if (t < cnt) tile(t, true, ks3, ks2, vs3, vs2, vs1), ++t;

        // ---- final PV of the last tile (its V sits in slot (cnt - 1) % 4)
        {
            const int r = (cnt - 1) & 3;
            const uint16_t *vr = r == 0 ? vs0 : (r == 1 ? vs1 : (r == 2 ? vs2 : vs3));
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int d = 32 * db + l32;
                    const int f = cc * 4 + db;
                    const bf16x8 vf =
                        f < kVPre ? vpre[f < kVPre ? f : 0]
                                  : *reinterpret_cast<const bf16x8 *>(vr + d * kBN +
                                                                      8 * v_pos(d, 2 * cc + hi));
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[cc], o[db], 0, 0, 0);
                }
            __builtin_amdgcn_s_setprio(0);
        }
        // no LDS-DMA may still be writing when the workgroup's LDS is released;
        // group 0 matches group 1's extra barrier
        PMA_WAIT_VM(0);
        if (grp == 0) PMA_PHASE_END(0);

        // ---- epilogue: O row = O^T column / row sum; register v of d-block db is
        // channel 32*db + 8*(v/4) + 4*hi + v%4
        const float lt = half_sum(lsum);
        if (part >= 0) {
            // a part: unnormalised O (reference mref) and the row sum, for the merge
            const int r = wave * 32 + l32;
            float *orow = pres + r * kD + 4 * hi;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 w = {o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
                    *reinterpret_cast<f32x4 *>(orow + 32 * db + 8 * g) = w;
                }
            if (hi == 0) {
                pres[kBM * kD + 2 * r] = mref;
                pres[kBM * kD + 2 * r + 1] = lt;
            }
            continue;
        }
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
    }   // work loop
    if (tid == 0) {
        uint64_t *st = ((kernarg_launch)__builtin_amdgcn_kernarg_segment_ptr())->stamps;
        if (st) {
            st[4 * blockIdx.x + 2] = __builtin_amdgcn_s_memtime();
            st[4 * blockIdx.x + 3] = __builtin_amdgcn_s_memrealtime();
        }
    }
}

// Zero the work-queue counters (a kernel rather than a memset, so the
// sequence can be captured in a graph and replayed).
__global__ void flash_queue_reset_kernel(int *queue) {
    if (threadIdx.x < 16) queue[threadIdx.x] = 0;
}

// Combine the parts of the split items: per row, m = max_p m_p and
// O = sum_p 2^(m_p - m) O_p / sum_p 2^(m_p - m) l_p (parts with l_p = 0 hold
// no key of the row's document and carry no weight).  One workgroup per
// split item and 8 rows; 32 threads per row, 4 channels each.
__global__ __launch_bounds__(256) void flash_merge_kernel(FlashLaunch a) {
    const int total = a.H * a.nqt;
    const int per_xcd = (total + 7) / 8;
    const int gi = (int)blockIdx.x / (kBM / 8), rb = (int)blockIdx.x % (kBM / 8);
    const int xcd = gi / a.split_items, s = gi % a.split_items;
    const int item = xcd * per_xcd + per_xcd - a.split_items + s;
    if (item >= total) return;
    const int head = item / a.nqt;
    const int qt = a.order[item % a.nqt];
    const int r = rb * 8 + (int)(threadIdx.x >> 5), c4 = (int)(threadIdx.x & 31);
    const int qrow = qt * kBM + r;
    if (qrow >= a.L) return;
    const float *base = a.part + (int64_t)gi * kMaxSplitParts * kPartFloats;
    const int nparts = split_parts(a);
    float mp[kMaxSplitParts], lp[kMaxSplitParts], m = -INFINITY;
#pragma unroll
    for (int p = 0; p < kMaxSplitParts; ++p) {
        mp[p] = -INFINITY;
        lp[p] = 0.f;
        if (p < nparts) {
            mp[p] = base[p * kPartFloats + kBM * kD + 2 * r];
            lp[p] = base[p * kPartFloats + kBM * kD + 2 * r + 1];
        }
        if (lp[p] > 0.f) m = fmaxf(m, mp[p]);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
#pragma unroll
    for (int p = 0; p < kMaxSplitParts; ++p) {
        if (!(lp[p] > 0.f)) continue;
        const float w = __builtin_amdgcn_exp2f(mp[p] - m);
        l = fmaf(w, lp[p], l);
        const f32x4 op = *reinterpret_cast<const f32x4 *>(base + p * kPartFloats + r * kD + 4 * c4);
        acc += w * op;
    }
    const float inv = 1.0f / l;
    uint2 wv;
    wv.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    wv.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2 *>(a.o + (int64_t)qrow * a.o_ld + head * kD + 4 * c4) = wv;
    if (a.lse && c4 == 0)
        a.lse[(int64_t)head * a.L + qrow] = (m + __log2f(l)) * 0.69314718055994531f;
}

}  // namespace

int32_t flash_split_items(int32_t H, int32_t L) {
    // below kSplitMinKeyTiles an item is short enough that the queue's fetch
    // and the parts' set-up cost more than the balance gains (measured: 1-10%
    // slower at 4096 keys, 1.6% faster at 8192 with 2 parts per split item,
    // 2-4% faster from 16384 with 4); 0 turns the queue off
    const int nqt = (L + kBM - 1) / kBM, nkt = (L + kBN - 1) / kBN;
    if (nkt < kSplitMinKeyTiles) return 0;
    const int per_xcd = (H * nqt + 7) / 8;
    return per_xcd < kSplitItems ? per_xcd : kSplitItems;
}

size_t flash_split_bytes_for(int32_t split_items) {
    return kFlashQueueBytes + (size_t)8 * split_items * kMaxSplitParts * kPartFloats * sizeof(float);
}

size_t flash_split_bytes(int32_t H, int32_t L) { return flash_split_bytes_for(flash_split_items(H, L)); }

void flash_tiles(int32_t *tile_m, int32_t *tile_n) {
    *tile_m = kBM;
    *tile_n = kBN;
}

int32_t flash_max_k_tiles() { return (kLdsBytes - kStaticLds) / 4 - 4; }

hipError_t launch_flash_attention(const FlashLaunch &a, hipStream_t s) {
    const int total = a.H * a.nqt;
    const int per_xcd = (total + 7) / 8;
    const size_t dyn = 4 * ((size_t)a.nkt + 4);
    if (!a.queue) {
        flash_fwd_kernel<<<8 * per_xcd, kNW * 64, dyn, s>>>(a);
        return hipGetLastError();
    }
    // persistent: one workgroup per CU (the LDS admits one)
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    FlashLaunch b = a;
    if (cus > kFlashStampGroups) b.stamps = nullptr;
    flash_queue_reset_kernel<<<1, 64, 0, s>>>(a.queue);
    flash_fwd_kernel<<<cus, kNW * 64, dyn, s>>>(b);
    if (a.split_items > 0) flash_merge_kernel<<<8 * a.split_items * (kBM / 8), 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace pma
