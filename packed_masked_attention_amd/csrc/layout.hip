// layout.hip -- packed layout validation, document ids and the tile map.
//
// Page "MiniMaxH3Transformer3DModel" (diffusers API page): forward parameters
// define the packed layout (token_tags 0 video / 1 text / 2 audio,
// position_ids (t, h, w), timestep_indices into the distinct timesteps, and
// the video/audio/text index tensors); the intro keeps rows tagged -1 in their
// own attention document through a boolean mask.  A row pair may attend iff
// both or neither row is padding, so a tile of the L x L mask is described by
// which documents its q rows and k rows contain: one 2-bit flag per row tile
// (bit 0: holds a non-padding row, bit 1: holds a padding row).
//
// Five small launches, all integer work and deterministic:
//   init   zero the counters and flags, reset the status word
//   rows   per-row checks, doc ids, per-tag row counts, row-tile flags
//   index  index-tensor checks (range, strictly ascending, tag agreement)
//   tiles  one wave per q-tile: class of every k-tile and the compacted list
//   order  one block: q-tiles ranked by (count desc, index asc); count checks
#include "internal.h"

#include <climits>

namespace pma {
namespace {

constexpr int kBlock = 256;

__global__ void layout_init_kernel(int32_t *scratch, int32_t n, int32_t *status) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) scratch[i] = 0;
    if (i == 0) {
        status[0] = 0;
        status[1] = INT_MAX;
    }
}

__global__ __launch_bounds__(kBlock) void layout_rows_kernel(LayoutLaunch a) {
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const bool in = i < a.L;
    int bits = 0, is_pad = 0, tag = 0;
    if (in) {
        tag = a.tags[i];
        if (!(tag == -1 || tag == 0 || tag == 1 || tag == 2)) bits |= PMA_LAYOUT_BAD_TAG;
        is_pad = (tag == -1);
        if (!is_pad) {
            int t = a.ts_idx[i];
            if (t < 0 || t >= a.T) bits |= PMA_LAYOUT_BAD_TIMESTEP;
        }
        for (int ax = 0; ax < 3; ++ax) {
            int p = a.pos[3 * (int64_t)i + ax];
            if (p <= -(1 << 24) || p >= (1 << 24)) bits |= PMA_LAYOUT_BAD_POSITION;
        }
        a.doc[i] = is_pad;
        if (bits) {
            atomicOr(&a.status[0], bits);
            atomicMin(&a.status[1], i);
        }
    }
    // per-tag row counts: one atomic per wave and tag
    int32_t *tag_count = a.scratch;
    for (int t = 0; t < 3; ++t) {
        uint64_t m = __ballot(in && tag == t);
        if ((threadIdx.x & 63) == 0 && m) atomicAdd(&tag_count[t], (int)__popcll(m));
    }
    // row-tile flags: a wave's 64 rows lie in one tile because tiles are
    // multiples of 64 rows and waves start on a multiple of 64
    uint64_t real = __ballot(in && !is_pad), pad = __ballot(in && is_pad);
    if ((threadIdx.x & 63) == 0 && (real | pad)) {
        int f = (real ? 1 : 0) | (pad ? 2 : 0);
        int row0 = i;  // lane 0's row
        int32_t *qflags = a.scratch + 3, *kflags = a.scratch + 3 + a.nqt;
        atomicOr(&qflags[row0 / a.tile_m], f);
        atomicOr(&kflags[row0 / a.tile_n], f);
    }
}

__global__ __launch_bounds__(kBlock) void layout_index_kernel(LayoutLaunch a) {
    const int g = blockIdx.x * kBlock + threadIdx.x;
    const int n_all = a.nv + a.na + a.nt;
    int bits = 0;
    if (g < n_all) {
        const int32_t *idx;
        int n, want, j;
        if (g < a.nv) { idx = a.vid; n = a.nv; want = 0; j = g; }
        else if (g < a.nv + a.na) { idx = a.aud; n = a.na; want = 2; j = g - a.nv; }
        else { idx = a.txt; n = a.nt; want = 1; j = g - a.nv - a.na; }
        (void)n;
        int r = idx[j];
        if (r < 0 || r >= a.L) {
            bits |= PMA_LAYOUT_BAD_INDEX;
        } else {
            if (j > 0 && !(idx[j - 1] < r)) bits |= PMA_LAYOUT_UNSORTED_INDEX;
            if (a.tags[r] != want) bits |= PMA_LAYOUT_INDEX_TAG;
        }
    }
    // OR across the wave, one atomic per wave
    for (int off = 32; off >= 1; off >>= 1) bits |= __shfl_xor(bits, off);
    if ((threadIdx.x & 63) == 0 && bits) atomicOr(&a.status[0], bits);
}

// One wave per q-tile; 4 q-tiles per block.
__global__ __launch_bounds__(kBlock) void layout_tiles_kernel(LayoutLaunch a) {
    const int lane = threadIdx.x & 63;
    const int qt = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    if (qt >= a.nqt) return;
    const int32_t *qflags = a.scratch + 3, *kflags = a.scratch + 3 + a.nqt;
    const int fq = qflags[qt];
    uint8_t *cls = a.cls + (int64_t)qt * a.nkt;
    int32_t *list = a.list + (int64_t)qt * a.nkt;
    int n = 0;
    for (int base = 0; base < a.nkt; base += 64) {
        const int kt = base + lane;
        int c = PMA_TILE_EMPTY;
        if (kt < a.nkt) {
            const int fk = kflags[kt];
            if (fq & fk) c = (fq == fk && fq != 3) ? PMA_TILE_FULL : PMA_TILE_PARTIAL;
            cls[kt] = (uint8_t)c;
        }
        const uint64_t nz = __ballot(c != PMA_TILE_EMPTY);
        if (c != PMA_TILE_EMPTY) {
            const int before = __popcll(nz & ((1ull << lane) - 1ull));
            list[n + before] = kt;
        }
        n += __popcll(nz);
    }
    for (int j = n + lane; j < a.nkt; j += 64) list[j] = -1;
    if (lane == 0) a.count[qt] = n;
}

__global__ __launch_bounds__(kBlock) void layout_order_kernel(LayoutLaunch a) {
    for (int q = threadIdx.x; q < a.nqt; q += kBlock) {
        const int cq = a.count[q];
        int rank = 0;
        for (int b = 0; b < a.nqt; ++b) {
            const int cb = a.count[b];
            rank += (cb > cq) || (cb == cq && b < q);
        }
        a.order[rank] = q;
    }
    if (threadIdx.x == 0) {
        const int32_t *tag_count = a.scratch;
        if (tag_count[0] != a.nv || tag_count[2] != a.na || tag_count[1] != a.nt)
            atomicOr(&a.status[0], PMA_LAYOUT_INDEX_COUNT);
        if (a.status[1] == INT_MAX) a.status[1] = -1;
    }
}

}  // namespace

hipError_t launch_layout_build(const LayoutLaunch &a, hipStream_t s) {
    const int nscratch = 3 + a.nqt + a.nkt;
    layout_init_kernel<<<(nscratch + kBlock - 1) / kBlock, kBlock, 0, s>>>(a.scratch, nscratch,
                                                                          a.status);
    layout_rows_kernel<<<(a.L + kBlock - 1) / kBlock, kBlock, 0, s>>>(a);
    const int n_all = a.nv + a.na + a.nt;
    if (n_all > 0) layout_index_kernel<<<(n_all + kBlock - 1) / kBlock, kBlock, 0, s>>>(a);
    layout_tiles_kernel<<<(a.nqt + 3) / 4, kBlock, 0, s>>>(a);
    layout_order_kernel<<<1, kBlock, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace pma
