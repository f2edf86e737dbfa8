// api.cpp -- the C ABI of libpma: host-side argument checks and launches.
// The operations and their page citations are documented in include/pma.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.h"

using namespace pma;

namespace {

thread_local char g_err[512] = "";

pma_status fail(pma_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

pma_status hip_fail(hipError_t e, const char *what) {
    return fail(PMA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

#define PMA_CHECK_HIP(expr, what)                   \
    do {                                            \
        hipError_t e_ = (expr);                     \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

bool aligned(const void *p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

// Per-device "is gfx950" cache.
std::mutex g_dev_mu;
int g_dev_ok[64];  // 0 unknown, 1 yes, -1 no

pma_status check_device() {
    int dev = 0;
    PMA_CHECK_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(PMA_ERR_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        PMA_CHECK_HIP(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties");
        g_dev_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        if (g_dev_ok[dev] < 0)
            return fail(PMA_ERR_UNSUPPORTED, "device %d is %s, libpma is built for gfx950", dev,
                        prop.gcnArchName);
    }
    if (g_dev_ok[dev] < 0) return fail(PMA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return PMA_OK;
}

bool valid_tile(int32_t t) { return t == 64 || t == 128 || t == 256; }

// Layout workspace: doc [L] i32 | status [2] i32 (+pad) | count [nqt] | order [nqt]
// | list [nqt*nkt] | scratch [3+nqt+nkt] | class [nqt*nkt] u8 -- each part 256-aligned.
struct LayoutParts {
    size_t doc, status, count, order, list, scratch, cls, total;
};
LayoutParts layout_parts(int32_t L, int32_t tm, int32_t tn) {
    const size_t nqt = (L + tm - 1) / tm, nkt = (L + tn - 1) / tn;
    LayoutParts p;
    size_t off = 0;
    p.doc = off;     off = round_up(off + 4 * (size_t)L, 256);
    p.status = off;  off = round_up(off + 8, 256);
    p.count = off;   off = round_up(off + 4 * nqt, 256);
    p.order = off;   off = round_up(off + 4 * nqt, 256);
    p.list = off;    off = round_up(off + 4 * nqt * nkt, 256);
    p.scratch = off; off = round_up(off + 4 * (3 + nqt + nkt), 256);
    p.cls = off;     off = round_up(off + nqt * nkt, 256);
    p.total = off;
    return p;
}

pma_status check_attn_params(const pma_attn_params *p) {
    if (!p) return fail(PMA_ERR_NULL, "attention params are NULL");
    if (p->head_dim != kHeadDim)
        return fail(PMA_ERR_UNSUPPORTED, "head_dim %d (only 128 is built)", p->head_dim);
    if (p->num_heads < 1 || p->num_heads > 4096)
        return fail(PMA_ERR_SHAPE, "num_heads %d", p->num_heads);
    if (!(p->rope_freq_dim == 8 || p->rope_freq_dim == 16))
        return fail(PMA_ERR_UNSUPPORTED, "rope_freq_dim %d (8 or 16)", p->rope_freq_dim);
    if (!(p->rope_theta > 0.f) || !std::isfinite(p->rope_theta))
        return fail(PMA_ERR_SHAPE, "rope_theta %g", (double)p->rope_theta);
    if (!(p->qk_norm_eps >= 0.f) || !std::isfinite(p->qk_norm_eps))
        return fail(PMA_ERR_SHAPE, "qk_norm_eps %g", (double)p->qk_norm_eps);
    if (!(p->softmax_scale >= 0.f) || !std::isfinite(p->softmax_scale))
        return fail(PMA_ERR_SHAPE, "softmax_scale %g", (double)p->softmax_scale);
    for (int a = 0; a < 3; ++a)
        if (!std::isfinite(p->pos_scale[a]))
            return fail(PMA_ERR_SHAPE, "pos_scale[%d] %g", a, (double)p->pos_scale[a]);
    return PMA_OK;
}

pma_status check_layout(const pma_layout *l) {
    if (!l) return fail(PMA_ERR_NULL, "layout is NULL");
    if (l->seq_len < 1 || !l->doc || !l->tile_class || !l->tile_count || !l->tile_list ||
        !l->tile_order || !l->position_ids)
        return fail(PMA_ERR_NULL, "layout is not built");
    return PMA_OK;
}

int32_t padded_len(int32_t L) { return (int32_t)round_up((size_t)L, kPadRows); }

pma_status check_tok_major(const char *name, const pma_bf16 *x, int64_t ld, int32_t H) {
    if (!x) return fail(PMA_ERR_NULL, "%s is NULL", name);
    if (ld < (int64_t)H * kHeadDim) return fail(PMA_ERR_SHAPE, "%s_ld %lld < H*D", name, (long long)ld);
    if (ld % 8 != 0 || !aligned(x, 16))
        return fail(PMA_ERR_ALIGN, "%s must be 16-byte aligned with ld %% 8 == 0", name);
    return PMA_OK;
}

}  // namespace

namespace pma {
pma_status api_fail(pma_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}
pma_status api_check_device() { return check_device(); }
pma_status api_check_attn_params(const pma_attn_params *p) { return check_attn_params(p); }
void api_fill_rope(const pma_attn_params *p, PrepLaunch &a) {
    for (int f = 0; f < 16; ++f)
        a.inv_freq[f] = f < p->rope_freq_dim
                            ? std::pow((double)p->rope_theta, -(double)f / (double)p->rope_freq_dim)
                            : 0.0;
    for (int ax = 0; ax < 3; ++ax)
        a.pos_scale[ax] = p->pos_scale[ax] == 0.f ? 1.0 : (double)p->pos_scale[ax];
}
// The attention operand Q' carries the logit scale: Q' = q_normed_rotated *
// softmax_scale * log2(e), so the attention kernel's scores are log2-unit
// logits straight out of the MFMA and exp2 applies with no multiply.
float api_q_operand_scale(const pma_attn_params *p) {
    const float scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)kHeadDim);
    return scale * 1.4426950408889634f;
}
pma_status api_check_layout(const pma_layout *l) { return check_layout(l); }
int32_t api_padded_len(int32_t L) { return padded_len(L); }
}  // namespace pma

extern "C" {

const char *pma_status_string(pma_status s) {
    switch (s) {
        case PMA_OK: return "PMA_OK";
        case PMA_ERR_NULL: return "PMA_ERR_NULL";
        case PMA_ERR_SHAPE: return "PMA_ERR_SHAPE";
        case PMA_ERR_ALIGN: return "PMA_ERR_ALIGN";
        case PMA_ERR_WORKSPACE: return "PMA_ERR_WORKSPACE";
        case PMA_ERR_LAYOUT: return "PMA_ERR_LAYOUT";
        case PMA_ERR_DEVICE: return "PMA_ERR_DEVICE";
        case PMA_ERR_UNSUPPORTED: return "PMA_ERR_UNSUPPORTED";
    }
    return "PMA_ERR_UNKNOWN";
}

const char *pma_last_error(void) { return g_err; }

pma_status pma_device_check(void) { return check_device(); }

// ------------------------------------------------------------------ layout

pma_status pma_layout_workspace_size(int32_t seq_len, int32_t tile_m, int32_t tile_n,
                                     size_t *bytes) {
    if (!bytes) return fail(PMA_ERR_NULL, "bytes is NULL");
    if (tile_m == 0 && tile_n == 0) flash_tiles(&tile_m, &tile_n);
    if (seq_len < 1 || seq_len > (1 << 24)) return fail(PMA_ERR_SHAPE, "seq_len %d", seq_len);
    if (!valid_tile(tile_m) || !valid_tile(tile_n))
        return fail(PMA_ERR_SHAPE, "tiles %d x %d (64, 128 or 256)", tile_m, tile_n);
    *bytes = layout_parts(seq_len, tile_m, tile_n).total;
    return PMA_OK;
}

pma_status pma_layout_build(const pma_layout_desc *d, int32_t tile_m, int32_t tile_n,
                            void *workspace, size_t workspace_bytes, void *stream,
                            pma_layout *out) {
    if (!d || !out) return fail(PMA_ERR_NULL, "desc or out is NULL");
    if (tile_m == 0 && tile_n == 0) flash_tiles(&tile_m, &tile_n);
    size_t need = 0;
    pma_status st = pma_layout_workspace_size(d->seq_len, tile_m, tile_n, &need);
    if (st != PMA_OK) return st;
    if (d->num_timesteps < 1) return fail(PMA_ERR_SHAPE, "num_timesteps %d", d->num_timesteps);
    if (!d->token_tags || !d->position_ids || !d->timestep_indices)
        return fail(PMA_ERR_NULL, "token_tags, position_ids and timestep_indices are required");
    if (d->num_video < 0 || d->num_audio < 0 || d->num_text < 0 ||
        (int64_t)d->num_video + d->num_audio + d->num_text > d->seq_len)
        return fail(PMA_ERR_SHAPE, "index counts %d/%d/%d for L=%d", d->num_video, d->num_audio,
                    d->num_text, d->seq_len);
    if ((d->num_video && !d->video_indices) || (d->num_audio && !d->audio_indices) ||
        (d->num_text && !d->text_indices))
        return fail(PMA_ERR_NULL, "an index tensor with a non-zero count is NULL");
    if (!workspace) return fail(PMA_ERR_NULL, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(PMA_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
        return fail(PMA_ERR_WORKSPACE, "layout workspace %zu < %zu bytes", workspace_bytes, need);
    if ((st = check_device()) != PMA_OK) return st;

    const LayoutParts p = layout_parts(d->seq_len, tile_m, tile_n);
    char *ws = static_cast<char *>(workspace);
    pma_layout l;
    memset(&l, 0, sizeof l);
    l.seq_len = d->seq_len;
    l.num_timesteps = d->num_timesteps;
    l.tile_m = tile_m;
    l.tile_n = tile_n;
    l.num_q_tiles = (d->seq_len + tile_m - 1) / tile_m;
    l.num_k_tiles = (d->seq_len + tile_n - 1) / tile_n;
    l.token_tags = d->token_tags;
    l.position_ids = d->position_ids;
    l.timestep_indices = d->timestep_indices;
    l.doc = reinterpret_cast<int32_t *>(ws + p.doc);
    l.status = reinterpret_cast<int32_t *>(ws + p.status);
    l.tile_count = reinterpret_cast<int32_t *>(ws + p.count);
    l.tile_order = reinterpret_cast<int32_t *>(ws + p.order);
    l.tile_list = reinterpret_cast<int32_t *>(ws + p.list);
    l.scratch = reinterpret_cast<int32_t *>(ws + p.scratch);
    l.tile_class = reinterpret_cast<uint8_t *>(ws + p.cls);

    LayoutLaunch a;
    a.L = d->seq_len; a.T = d->num_timesteps; a.tile_m = tile_m; a.tile_n = tile_n;
    a.nqt = l.num_q_tiles; a.nkt = l.num_k_tiles;
    a.tags = d->token_tags; a.pos = d->position_ids; a.ts_idx = d->timestep_indices;
    a.vid = d->video_indices; a.aud = d->audio_indices; a.txt = d->text_indices;
    a.nv = d->num_video; a.na = d->num_audio; a.nt = d->num_text;
    a.doc = l.doc; a.cls = l.tile_class; a.count = l.tile_count; a.list = l.tile_list;
    a.order = l.tile_order; a.status = l.status; a.scratch = l.scratch;
    PMA_CHECK_HIP(launch_layout_build(a, static_cast<hipStream_t>(stream)), "layout launch");
    *out = l;
    return PMA_OK;
}

pma_status pma_layout_read_status(const pma_layout *layout, void *stream, int32_t *bits,
                                  int32_t *first_bad_row) {
    if (!layout || !layout->status) return fail(PMA_ERR_NULL, "layout is not built");
    int32_t h[2] = {0, -1};
    hipStream_t s = static_cast<hipStream_t>(stream);
    PMA_CHECK_HIP(hipMemcpyAsync(h, layout->status, sizeof h, hipMemcpyDeviceToHost, s),
                  "status copy");
    PMA_CHECK_HIP(hipStreamSynchronize(s), "status sync");
    if (bits) *bits = h[0];
    if (first_bad_row) *first_bad_row = h[1];
    if (h[0] != 0)
        return fail(PMA_ERR_LAYOUT, "layout status bits 0x%x, first bad row %d", h[0], h[1]);
    return PMA_OK;
}

// --------------------------------------------------------------- attention

pma_status pma_attention_tiles(int32_t *tile_m, int32_t *tile_n) {
    if (!tile_m || !tile_n) return fail(PMA_ERR_NULL, "NULL output");
    flash_tiles(tile_m, tile_n);
    return PMA_OK;
}

pma_status pma_attention_padded_len(int32_t seq_len, int32_t *out) {
    if (!out) return fail(PMA_ERR_NULL, "NULL output");
    if (seq_len < 1 || seq_len > (1 << 24)) return fail(PMA_ERR_SHAPE, "seq_len %d", seq_len);
    *out = padded_len(seq_len);
    return PMA_OK;
}

pma_status pma_qk_norm_rope(const pma_attn_params *p, const pma_layout *layout,
                            const pma_bf16 *q, int64_t q_ld, const pma_bf16 *k, int64_t k_ld,
                            const pma_bf16 *v, int64_t v_ld, const float *q_norm_weight,
                            const float *k_norm_weight, pma_bf16 *qh, pma_bf16 *kh,
                            pma_bf16 *vt, void *stream) {
    pma_status st;
    if ((st = check_attn_params(p)) != PMA_OK) return st;
    if ((st = check_layout(layout)) != PMA_OK) return st;
    const int32_t H = p->num_heads;
    if ((st = check_tok_major("q", q, q_ld, H)) != PMA_OK) return st;
    if ((st = check_tok_major("k", k, k_ld, H)) != PMA_OK) return st;
    if ((st = check_tok_major("v", v, v_ld, H)) != PMA_OK) return st;
    if (!q_norm_weight || !k_norm_weight || !qh || !kh || !vt)
        return fail(PMA_ERR_NULL, "norm weights and outputs are required");
    if (!aligned(q_norm_weight, 16) || !aligned(k_norm_weight, 16) || !aligned(qh, 16) ||
        !aligned(kh, 16) || !aligned(vt, 16))
        return fail(PMA_ERR_ALIGN, "norm weights and outputs must be 16-byte aligned");
    if ((st = check_device()) != PMA_OK) return st;

    PrepLaunch a;
    a.L = layout->seq_len;
    a.Lp = padded_len(a.L);
    a.H = H;
    a.F = p->rope_freq_dim;
    a.eps = p->qk_norm_eps;
    a.qscale = api_q_operand_scale(p);
    api_fill_rope(p, a);
    a.q = q; a.k = k; a.v = v;
    a.q_ld = q_ld; a.k_ld = k_ld; a.v_ld = v_ld;
    a.wq = q_norm_weight; a.wk = k_norm_weight;
    a.pos = layout->position_ids;
    a.qh = qh; a.kh = kh; a.vt = vt;
    PMA_CHECK_HIP(launch_qk_norm_rope(a, static_cast<hipStream_t>(stream)), "qk_norm_rope launch");
    return PMA_OK;
}

pma_status pma_flash_workspace_size(const pma_attn_params *p, int32_t seq_len, size_t *bytes) {
    pma_status st;
    if ((st = check_attn_params(p)) != PMA_OK) return st;
    if (!bytes) return fail(PMA_ERR_NULL, "bytes is NULL");
    if (seq_len < 1 || seq_len > (1 << 24)) return fail(PMA_ERR_SHAPE, "seq_len %d", seq_len);
    // the clock stamps of the persistent launch follow the partial results
    *bytes = flash_split_bytes(p->num_heads, seq_len) +
             (flash_split_items(p->num_heads, seq_len) > 0 ? kFlashStampBytes : 0);
    return PMA_OK;
}

}  // extern "C"

namespace {

// Argument checks shared by the two flash entry points.
pma_status check_flash_args(const pma_attn_params *p, const pma_layout *layout,
                            const pma_bf16 *qh, const pma_bf16 *kh, const pma_bf16 *vt,
                            pma_bf16 *o, int64_t o_ld, float *lse) {
    pma_status st;
    if ((st = check_attn_params(p)) != PMA_OK) return st;
    if ((st = check_layout(layout)) != PMA_OK) return st;
    int32_t tm, tn;
    flash_tiles(&tm, &tn);
    if (layout->tile_m != tm || layout->tile_n != tn)
        return fail(PMA_ERR_SHAPE, "layout tiles %d x %d, the attention kernel needs %d x %d",
                    layout->tile_m, layout->tile_n, tm, tn);
    if (layout->num_k_tiles > flash_max_k_tiles())
        return fail(PMA_ERR_SHAPE, "seq_len %d: the attention kernel takes at most %d k-tiles (%d keys)",
                    layout->seq_len, flash_max_k_tiles(), flash_max_k_tiles() * tn);
    if (!qh || !kh || !vt) return fail(PMA_ERR_NULL, "qh, kh and vt are required");
    if (!aligned(qh, 16) || !aligned(kh, 16) || !aligned(vt, 16))
        return fail(PMA_ERR_ALIGN, "qh, kh, vt must be 16-byte aligned");
    if ((st = check_tok_major("o", o, o_ld, p->num_heads)) != PMA_OK) return st;
    if (lse && !aligned(lse, 4)) return fail(PMA_ERR_ALIGN, "lse must be 4-byte aligned");
    return PMA_OK;
}

// Launch with split_items split items per XCD (0: one item per workgroup,
// no work queue); ws holds flash_split_bytes_for(split_items) bytes, then
// (stamps) the clock-stamp area.
pma_status flash_launch(const pma_attn_params *p, const pma_layout *layout, const pma_bf16 *qh,
                        const pma_bf16 *kh, const pma_bf16 *vt, pma_bf16 *o, int64_t o_ld,
                        float *lse, void *ws, int32_t split_items, bool stamps, void *stream) {
    FlashLaunch a;
    a.L = layout->seq_len;
    a.Lp = padded_len(a.L);
    a.H = p->num_heads;
    a.nqt = layout->num_q_tiles;
    a.nkt = layout->num_k_tiles;
    a.qh = qh; a.kh = kh; a.vt = vt;
    a.o = o; a.o_ld = o_ld; a.lse = lse;
    a.doc = layout->doc;
    a.cls = layout->tile_class;
    a.count = layout->tile_count;
    a.list = layout->tile_list;
    a.order = layout->tile_order;
    a.split_items = split_items;
    a.queue = split_items > 0 ? static_cast<int32_t *>(ws) : nullptr;
    a.part = split_items > 0 ? reinterpret_cast<float *>(static_cast<char *>(ws) + kFlashQueueBytes)
                             : nullptr;
    a.stamps = split_items > 0 && stamps
                   ? reinterpret_cast<uint64_t *>(static_cast<char *>(ws) +
                                                  flash_split_bytes_for(split_items))
                   : nullptr;
    PMA_CHECK_HIP(launch_flash_attention(a, static_cast<hipStream_t>(stream)), "flash launch");
    return PMA_OK;
}

// ---- scratch of the allocation-free entry point.  A file-scope device
// array: every GPU the library runs on holds its own copy (at its own
// address) until the process ends.  Host code never uses the array's name
// as an address: the device address is fetched once per device with
// hipGetSymbolAddress and kept in g_scratch.
constexpr size_t kScratchBytes = PMA_FLASH_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch[64];

pma_status scratch_address(void **out) {
    int dev = 0;
    PMA_CHECK_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(PMA_ERR_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        PMA_CHECK_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(PMA_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return PMA_OK;
}

}  // namespace

extern "C" {

pma_status pma_flash_attention(const pma_attn_params *p, const pma_layout *layout,
                               const pma_bf16 *qh, const pma_bf16 *kh, const pma_bf16 *vt,
                               pma_bf16 *o, int64_t o_ld, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream) {
    pma_status st;
    if ((st = check_flash_args(p, layout, qh, kh, vt, o, o_ld, lse)) != PMA_OK) return st;
    if (workspace) {
        size_t need = 0;
        if ((st = pma_flash_workspace_size(p, layout->seq_len, &need)) != PMA_OK) return st;
        if (!aligned(workspace, 256)) return fail(PMA_ERR_ALIGN, "workspace must be 256-byte aligned");
        if (workspace_bytes < need)
            return fail(PMA_ERR_WORKSPACE, "flash workspace %zu < %zu bytes", workspace_bytes, need);
    }
    if ((st = check_device()) != PMA_OK) return st;
    // the work queue pays off on long key lists only (see flash_split_items)
    const int32_t split = workspace ? flash_split_items(p->num_heads, layout->seq_len) : 0;
    return flash_launch(p, layout, qh, kh, vt, o, o_ld, lse, workspace, split, true, stream);
}

pma_status pma_flash_attention_static(const pma_attn_params *p, const pma_layout *layout,
                                      const pma_bf16 *qh, const pma_bf16 *kh, const pma_bf16 *vt,
                                      pma_bf16 *o, int64_t o_ld, float *lse, void *stream) {
    pma_status st;
    if ((st = check_flash_args(p, layout, qh, kh, vt, o, o_ld, lse)) != PMA_OK) return st;
    if ((st = check_device()) != PMA_OK) return st;
    // as many split items per XCD as the workspace form would take, up to
    // what the array holds
    int32_t split = flash_split_items(p->num_heads, layout->seq_len);
    while (split > 0 && flash_split_bytes_for(split) > kScratchBytes) --split;
    const size_t need = flash_split_bytes_for(split);
    if (need > kScratchBytes)
        return fail(PMA_ERR_WORKSPACE, "flash scratch needs %zu bytes, the static array holds %zu",
                    need, kScratchBytes);
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != PMA_OK) return st;
    return flash_launch(p, layout, qh, kh, vt, o, o_ld, lse, ws, split, false, stream);
}

pma_status pma_attention_workspace_size(const pma_attn_params *p, int32_t seq_len,
                                        size_t *bytes) {
    pma_status st;
    if ((st = check_attn_params(p)) != PMA_OK) return st;
    if (!bytes) return fail(PMA_ERR_NULL, "bytes is NULL");
    if (seq_len < 1 || seq_len > (1 << 24)) return fail(PMA_ERR_SHAPE, "seq_len %d", seq_len);
    const size_t one = round_up((size_t)p->num_heads * padded_len(seq_len) * kHeadDim * 2, 256);
    size_t flash = 0;
    if ((st = pma_flash_workspace_size(p, seq_len, &flash)) != PMA_OK) return st;
    *bytes = 3 * one + flash;
    return PMA_OK;
}

pma_status pma_attention(const pma_attn_params *p, const pma_layout *layout, const pma_bf16 *q,
                         int64_t q_ld, const pma_bf16 *k, int64_t k_ld, const pma_bf16 *v,
                         int64_t v_ld, const float *q_norm_weight, const float *k_norm_weight,
                         pma_bf16 *o, int64_t o_ld, float *lse, void *workspace,
                         size_t workspace_bytes, void *stream) {
    pma_status st;
    if ((st = check_layout(layout)) != PMA_OK) return st;
    size_t need = 0;
    if ((st = pma_attention_workspace_size(p, layout->seq_len, &need)) != PMA_OK) return st;
    if (!workspace) return fail(PMA_ERR_NULL, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(PMA_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
        return fail(PMA_ERR_WORKSPACE, "attention workspace %zu < %zu bytes", workspace_bytes, need);
    const size_t one = round_up((size_t)p->num_heads * padded_len(layout->seq_len) * kHeadDim * 2, 256);
    pma_bf16 *qh = static_cast<pma_bf16 *>(workspace);
    pma_bf16 *kh = reinterpret_cast<pma_bf16 *>(static_cast<char *>(workspace) + one);
    pma_bf16 *vt = reinterpret_cast<pma_bf16 *>(static_cast<char *>(workspace) + 2 * one);
    if ((st = pma_qk_norm_rope(p, layout, q, q_ld, k, k_ld, v, v_ld, q_norm_weight, k_norm_weight,
                               qh, kh, vt, stream)) != PMA_OK)
        return st;
    return pma_flash_attention(p, layout, qh, kh, vt, o, o_ld, lse,
                               static_cast<char *>(workspace) + 3 * one, need - 3 * one, stream);
}

}  // extern "C"
