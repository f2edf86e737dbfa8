// io_api.cpp -- C ABI of the input and output path (timestep MLP, row pack,
// output heads): argument checks and launches.  The operations and their page
// citations are documented in include/pma.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "internal.h"

using namespace pma;

namespace pma {
pma_status api_fail(pma_status s, const char *fmt, ...);
pma_status api_check_device();
}  // namespace pma

namespace {

bool aligned(const void *p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

#define FAIL(...) return pma::api_fail(__VA_ARGS__)
#define CHECK_HIP(expr, what)                                                             \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess) FAIL(PMA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e_)); \
    } while (0)

// K ranges of the head GEMM: the fewest (a divisor of hidden / chunk, so
// every range is whole LDS chunks) that give about 2048 waves of 32 rows.
int head_splits(int32_t rows, int32_t hidden) {
    const int steps = hidden / head_k_chunk();
    const int tiles = (rows + 31) / 32;
    for (int d = 1; d <= steps; ++d)
        if (steps % d == 0 && (int64_t)tiles * d >= 2048) return d;
    return steps;
}

pma_status check_io_params(const pma_io_params *p) {
    if (!p) FAIL(PMA_ERR_NULL, "io params are NULL");
    if (p->hidden < 128 || p->hidden % 128 != 0 || p->hidden > head_max_hidden())
        FAIL(PMA_ERR_SHAPE, "hidden %d (multiple of 128, <= %d)", p->hidden, head_max_hidden());
    if (p->video_channels < 32 || p->video_channels % 32 != 0 || p->audio_channels < 32 ||
        p->audio_channels % 32 != 0)
        FAIL(PMA_ERR_SHAPE, "video_channels %d / audio_channels %d (multiples of 32)",
             p->video_channels, p->audio_channels);
    if (p->video_out < 32 || p->video_out % 32 != 0 || p->video_out > head_max_out() ||
        p->audio_out < 32 || p->audio_out % 32 != 0 || p->audio_out > head_max_out())
        FAIL(PMA_ERR_SHAPE, "video_out %d / audio_out %d (multiples of 32, <= %d)", p->video_out,
             p->audio_out, head_max_out());
    if (p->time_embed_dim < 4 || p->time_embed_dim % 4 != 0)
        FAIL(PMA_ERR_SHAPE, "time_embed_dim %d (multiple of 4)", p->time_embed_dim);
    if (!(p->final_norm_eps >= 0.f)) FAIL(PMA_ERR_SHAPE, "final_norm_eps %g", (double)p->final_norm_eps);
    return PMA_OK;
}

pma_status check_desc(const pma_layout_desc *d) {
    if (!d) FAIL(PMA_ERR_NULL, "layout descriptor is NULL");
    if (d->seq_len < 1 || d->num_timesteps < 1)
        FAIL(PMA_ERR_SHAPE, "seq_len %d, num_timesteps %d", d->seq_len, d->num_timesteps);
    if (d->num_video < 0 || d->num_audio < 0 || d->num_text < 0 ||
        (int64_t)d->num_video + d->num_audio + d->num_text > d->seq_len)
        FAIL(PMA_ERR_SHAPE, "row counts %d + %d + %d exceed seq_len %d", d->num_video,
             d->num_audio, d->num_text, d->seq_len);
    if ((d->num_video && !d->video_indices) || (d->num_audio && !d->audio_indices) ||
        (d->num_text && !d->text_indices))
        FAIL(PMA_ERR_NULL, "an index array with a non-zero count is NULL");
    return PMA_OK;
}

// head workspace: stats [rows] float2 | partial [splits][rows][nout] fp32, per head, 256-aligned
struct HeadParts {
    size_t stats_v, part_v, stats_a, part_a, total;
};
HeadParts head_parts(const pma_io_params *p, int32_t nv, int32_t na) {
    HeadParts h;
    size_t off = 0;
    h.stats_v = off; off = round_up(off + 8 * (size_t)nv, 256);
    h.part_v = off;
    off = round_up(off + 4 * (size_t)head_splits(nv, p->hidden) * nv * p->video_out, 256);
    h.stats_a = off; off = round_up(off + 8 * (size_t)na, 256);
    h.part_a = off;
    off = round_up(off + 4 * (size_t)head_splits(na, p->hidden) * na * p->audio_out, 256);
    h.total = off;
    return h;
}

}  // namespace

extern "C" {

pma_status pma_timestep_embed(const pma_temb_params *p, int32_t T, const float *timestep,
                              const float *w1, const float *b1, const float *w2,
                              const float *b2, float *inner, float *temb, pma_bf16 *temb_bf16,
                              void *stream) {
    if (!p) FAIL(PMA_ERR_NULL, "timestep params are NULL");
    if (p->freq_dim < 4 || p->freq_dim % 4 != 0 || p->freq_dim > 2048)
        FAIL(PMA_ERR_SHAPE, "freq_dim %d (multiple of 4, 4..2048)", p->freq_dim);
    if (p->inner_dim < 4 || p->inner_dim % 4 != 0 || p->embed_dim < 4 || p->embed_dim % 4 != 0)
        FAIL(PMA_ERR_SHAPE, "inner_dim %d / embed_dim %d (multiples of 4)", p->inner_dim,
             p->embed_dim);
    if (!(p->max_period > 1.f)) FAIL(PMA_ERR_SHAPE, "max_period %g", (double)p->max_period);
    if (T < 1 || T > gemv_max_t()) FAIL(PMA_ERR_SHAPE, "num_timesteps %d (1..%d)", T, gemv_max_t());
    if (!timestep || !w1 || !b1 || !w2 || !b2 || !inner || !temb)
        FAIL(PMA_ERR_NULL, "timestep, weights, biases, inner and temb are required");
    if (!aligned(w1, 16) || !aligned(w2, 16) || !aligned(inner, 16) || !aligned(temb, 4) ||
        !aligned(timestep, 4) || !aligned(b1, 4) || !aligned(b2, 4) ||
        (temb_bf16 && !aligned(temb_bf16, 2)))
        FAIL(PMA_ERR_ALIGN, "w1, w2 and inner must be 16-byte aligned");
    pma_status st;
    if ((st = api_check_device()) != PMA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    GemvLaunch a{};
    a.T = T;
    a.K = p->freq_dim;
    a.N = p->inner_dim;
    a.group_rows = p->inner_dim;
    a.timestep = timestep;
    a.log_max_period = std::log((double)p->max_period);
    a.W = w1;
    a.b = b1;
    a.silu = 1;
    a.out = inner;
    CHECK_HIP(launch_gemv(a, s), "timestep MLP layer 1");
    GemvLaunch c{};
    c.T = T;
    c.K = p->inner_dim;
    c.N = p->embed_dim;
    c.group_rows = p->embed_dim;
    c.x = inner;
    c.W = w2;
    c.b = b2;
    c.out = temb;
    c.out_bf16 = temb_bf16;
    CHECK_HIP(launch_gemv(c, s), "timestep MLP layer 2");
    return PMA_OK;
}

pma_status pma_pack_rows(const pma_io_params *p, const pma_layout_desc *desc,
                         const float *video_rows, const float *w_video, const float *b_video,
                         const float *audio_rows, const float *w_audio, const float *b_audio,
                         const pma_bf16 *text_rows, int64_t text_ld, pma_bf16 *x,
                         void *stream) {
    pma_status st;
    if ((st = check_io_params(p)) != PMA_OK) return st;
    if ((st = check_desc(desc)) != PMA_OK) return st;
    if (!x) FAIL(PMA_ERR_NULL, "x is required");
    if (desc->num_video && (!video_rows || !w_video || !b_video))
        FAIL(PMA_ERR_NULL, "video rows, weight and bias are required");
    if (desc->num_audio && (!audio_rows || !w_audio || !b_audio))
        FAIL(PMA_ERR_NULL, "audio rows, weight and bias are required");
    if (desc->num_text && !text_rows) FAIL(PMA_ERR_NULL, "text rows are required");
    if (desc->num_text && (text_ld < p->hidden || text_ld % 8 != 0))
        FAIL(PMA_ERR_SHAPE, "text_ld %lld (>= hidden, multiple of 8)", (long long)text_ld);
    if (!aligned(x, 16) || (video_rows && !aligned(video_rows, 16)) ||
        (w_video && !aligned(w_video, 16)) || (audio_rows && !aligned(audio_rows, 16)) ||
        (w_audio && !aligned(w_audio, 16)) || (text_rows && !aligned(text_rows, 16)) ||
        (b_video && !aligned(b_video, 16)) || (b_audio && !aligned(b_audio, 16)))
        FAIL(PMA_ERR_ALIGN, "x, rows and weights must be 16-byte aligned");
    if ((st = api_check_device()) != PMA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t counts[2] = {desc->num_video, desc->num_audio};
    const int32_t chans[2] = {p->video_channels, p->audio_channels};
    const float *rows[2] = {video_rows, audio_rows};
    const float *ws[2] = {w_video, w_audio};
    const float *bs[2] = {b_video, b_audio};
    const int32_t *idx[2] = {desc->video_indices, desc->audio_indices};
    for (int m = 0; m < 2; ++m) {
        if (counts[m] == 0) continue;
        ProjLaunch a{};
        a.rows = counts[m];
        a.K = chans[m];
        a.N = p->hidden;
        a.L = desc->seq_len;
        a.X = rows[m];
        a.W = ws[m];
        a.b = bs[m];
        a.idx = idx[m];
        a.out = x;
        a.ld_out = p->hidden;
        CHECK_HIP(launch_proj_scatter(a, s), "input projection");
    }
    if (desc->num_text) {
        TextScatterLaunch t{};
        t.rows = desc->num_text;
        t.hidden = p->hidden;
        t.L = desc->seq_len;
        t.src = text_rows;
        t.ld_src = text_ld;
        t.idx = desc->text_indices;
        t.out = x;
        t.ld_out = p->hidden;
        CHECK_HIP(launch_text_scatter(t, s), "text scatter");
    }
    return PMA_OK;
}

pma_status pma_head_table(const pma_io_params *p, int32_t T, const float *temb,
                          const float *w_mod, float *table, void *stream) {
    pma_status st;
    if ((st = check_io_params(p)) != PMA_OK) return st;
    if (T < 1 || T > gemv_max_t()) FAIL(PMA_ERR_SHAPE, "num_timesteps %d (1..%d)", T, gemv_max_t());
    if (!temb || !w_mod || !table) FAIL(PMA_ERR_NULL, "temb, w_mod and table are required");
    if (!aligned(temb, 16) || !aligned(w_mod, 16) || !aligned(table, 4))
        FAIL(PMA_ERR_ALIGN, "temb and w_mod must be 16-byte aligned");
    if ((st = api_check_device()) != PMA_OK) return st;
    GemvLaunch a{};
    a.T = T;
    a.K = p->time_embed_dim;
    a.N = 4 * p->hidden;
    a.group_rows = 2 * p->hidden;
    a.x = temb;
    a.W = w_mod;
    a.out = table;
    CHECK_HIP(launch_gemv(a, static_cast<hipStream_t>(stream)), "head table");
    return PMA_OK;
}

pma_status pma_unpack_workspace_size(const pma_io_params *p, int32_t nv, int32_t na,
                                     size_t *bytes) {
    pma_status st;
    if ((st = check_io_params(p)) != PMA_OK) return st;
    if (!bytes) FAIL(PMA_ERR_NULL, "bytes is NULL");
    if (nv < 0 || na < 0) FAIL(PMA_ERR_SHAPE, "row counts %d, %d", nv, na);
    *bytes = head_parts(p, nv, na).total;
    return PMA_OK;
}

pma_status pma_unpack_rows(const pma_io_params *p, const pma_layout_desc *desc,
                           const pma_bf16 *x, const float *table, const float *w_video_out,
                           const float *b_video_out, const float *w_audio_out,
                           const float *b_audio_out, float *video_out, float *audio_out,
                           void *workspace, size_t workspace_bytes, void *stream) {
    pma_status st;
    if ((st = check_io_params(p)) != PMA_OK) return st;
    if ((st = check_desc(desc)) != PMA_OK) return st;
    if (!desc->timestep_indices) FAIL(PMA_ERR_NULL, "timestep_indices are required");
    if (desc->num_timesteps > head_max_t())
        FAIL(PMA_ERR_SHAPE, "num_timesteps %d (<= %d)", desc->num_timesteps, head_max_t());
    if (!x || !table) FAIL(PMA_ERR_NULL, "x and table are required");
    if (desc->num_video && (!w_video_out || !b_video_out || !video_out))
        FAIL(PMA_ERR_NULL, "video head weight, bias and output are required");
    if (desc->num_audio && (!w_audio_out || !b_audio_out || !audio_out))
        FAIL(PMA_ERR_NULL, "audio head weight, bias and output are required");
    const HeadParts hp = head_parts(p, desc->num_video, desc->num_audio);
    if (!workspace && hp.total) FAIL(PMA_ERR_NULL, "workspace is required");
    if (workspace_bytes < hp.total)
        FAIL(PMA_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, hp.total);
    if (!aligned(x, 16) || !aligned(table, 16) || (w_video_out && !aligned(w_video_out, 16)) ||
        (w_audio_out && !aligned(w_audio_out, 16)) || (video_out && !aligned(video_out, 4)) ||
        (audio_out && !aligned(audio_out, 4)) || (b_video_out && !aligned(b_video_out, 4)) ||
        (b_audio_out && !aligned(b_audio_out, 4)) || (workspace && !aligned(workspace, 256)))
        FAIL(PMA_ERR_ALIGN, "x, table and head weights 16-byte aligned, workspace 256-byte");
    if ((st = api_check_device()) != PMA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    for (int m = 0; m < 2; ++m) {
        HeadLaunch a{};
        a.rows = m ? desc->num_audio : desc->num_video;
        if (a.rows == 0) continue;
        a.hidden = p->hidden;
        a.nout = m ? p->audio_out : p->video_out;
        a.L = desc->seq_len;
        a.T = desc->num_timesteps;
        a.head = m;
        a.splits = head_splits(a.rows, p->hidden);
        a.eps = p->final_norm_eps;
        a.x = x;
        a.ld_x = p->hidden;
        a.idx = m ? desc->audio_indices : desc->video_indices;
        a.ts_idx = desc->timestep_indices;
        a.table = table;
        a.W = m ? w_audio_out : w_video_out;
        a.b = m ? b_audio_out : b_video_out;
        a.stats = reinterpret_cast<float2 *>(ws + (m ? hp.stats_a : hp.stats_v));
        a.partial = reinterpret_cast<float *>(ws + (m ? hp.part_a : hp.part_v));
        a.out = m ? audio_out : video_out;
        CHECK_HIP(launch_head(a, s), m ? "audio head" : "video head");
    }
    return PMA_OK;
}

}  // extern "C"
