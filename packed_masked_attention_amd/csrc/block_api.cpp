// block_api.cpp -- C ABI of the DiT block pieces: argument checks and launches.
// The operations and their page citations are documented in include/pma.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"

using namespace pma;

// shared with api.cpp
namespace pma {
pma_status api_fail(pma_status s, const char *fmt, ...);
pma_status api_check_device();
pma_status api_check_attn_params(const pma_attn_params *p);
pma_status api_check_layout(const pma_layout *l);
int32_t api_padded_len(int32_t L);
void api_fill_rope(const pma_attn_params *p, PrepLaunch &a);
float api_q_operand_scale(const pma_attn_params *p);
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

pma_status check_block_params(const pma_block_params *p) {
    if (!p) FAIL(PMA_ERR_NULL, "block params are NULL");
    pma_status st = api_check_attn_params(&p->attn);
    if (st != PMA_OK) return st;
    if (p->hidden < 256 || p->hidden % 256 != 0 || p->hidden > ln_modulate_max_hidden())
        FAIL(PMA_ERR_SHAPE, "hidden %d (multiple of 256, <= %d)", p->hidden,
             ln_modulate_max_hidden());
    if (p->ffn_dim < 128 || p->ffn_dim % 128 != 0) FAIL(PMA_ERR_SHAPE, "ffn_dim %d", p->ffn_dim);
    if (p->time_embed_dim < 8 || p->time_embed_dim % 8 != 0)
        FAIL(PMA_ERR_SHAPE, "time_embed_dim %d", p->time_embed_dim);
    if ((p->attn.num_heads * kHeadDim) % 256 != 0)
        FAIL(PMA_ERR_SHAPE, "num_heads * 128 = %d is not a multiple of 256",
             p->attn.num_heads * kHeadDim);
    if (!(p->norm_eps >= 0.f)) FAIL(PMA_ERR_SHAPE, "norm_eps %g", (double)p->norm_eps);
    return PMA_OK;
}

bool fits32(int64_t rows, int64_t ld) { return rows * ld * 2 < (int64_t)1 << 31; }

}  // namespace

extern "C" {

pma_status pma_adaln_table(const pma_block_params *p, int32_t T, const pma_bf16 *temb,
                           const pma_bf16 *w_ada, float *table, void *stream) {
    pma_status st;
    if ((st = check_block_params(p)) != PMA_OK) return st;
    if (T < 1 || T > adaln_max_t() || (int64_t)T * p->time_embed_dim > 24576)
        FAIL(PMA_ERR_SHAPE, "num_timesteps %d (1..%d, T*E <= 24576)", T, adaln_max_t());
    if (!temb || !w_ada || !table) FAIL(PMA_ERR_NULL, "temb, w_ada and table are required");
    if (!aligned(temb, 16) || !aligned(w_ada, 16) || !aligned(table, 4))
        FAIL(PMA_ERR_ALIGN, "temb and w_ada must be 16-byte aligned");
    if ((st = api_check_device()) != PMA_OK) return st;
    AdaLnLaunch a{T, p->time_embed_dim, p->hidden, temb, w_ada, table};
    CHECK_HIP(launch_adaln_table(a, static_cast<hipStream_t>(stream)), "adaln launch");
    return PMA_OK;
}

pma_status pma_ln_modulate(const pma_block_params *p, const pma_layout *layout,
                           const float *table, int32_t which, const pma_bf16 *x, pma_bf16 *out,
                           void *stream) {
    pma_status st;
    if ((st = check_block_params(p)) != PMA_OK) return st;
    if (!layout || !layout->token_tags || !layout->timestep_indices)
        FAIL(PMA_ERR_NULL, "layout is not built");
    if (!table || !x || !out) FAIL(PMA_ERR_NULL, "table, x and out are required");
    if (which != 0 && which != 1) FAIL(PMA_ERR_SHAPE, "which %d (0 or 1)", which);
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(table, 16))
        FAIL(PMA_ERR_ALIGN, "x, out and table must be 16-byte aligned");
    if ((st = api_check_device()) != PMA_OK) return st;
    LnModLaunch a;
    a.L = layout->seq_len;
    a.hidden = p->hidden;
    a.T = layout->num_timesteps;
    a.shift_chunk = which ? 3 : 0;
    a.eps = p->norm_eps;
    a.x = x;
    a.out = out;
    a.table = table;
    a.tags = layout->token_tags;
    a.ts_idx = layout->timestep_indices;
    a.stats = nullptr;
    a.stats_groups = a.stats_gw = 0;
    CHECK_HIP(launch_ln_modulate(a, static_cast<hipStream_t>(stream)), "ln_modulate launch");
    return PMA_OK;
}

}  // extern "C"

namespace {

// pma_linear; with stats (GATE_RESIDUAL only) the epilogue also writes the
// rounded rows' statistics, stats_groups pairs per row.
pma_status linear_impl(const pma_linear_args *g, float2 *stats, int32_t stats_groups, void *stream) {
    if (!g) FAIL(PMA_ERR_NULL, "args are NULL");
    if (g->epilogue < PMA_EPI_STORE || g->epilogue > PMA_EPI_SWIGLU)
        FAIL(PMA_ERR_SHAPE, "epilogue %d", g->epilogue);
    const int tn = g->epilogue == PMA_EPI_SWIGLU ? 128 : 256;
    if (g->M < 1 || g->N < tn || g->N % tn != 0 || g->K < 64 || g->K % 64 != 0)
        FAIL(PMA_ERR_SHAPE, "M=%d N=%d K=%d (N %% %d == 0, K %% 64 == 0)", g->M, g->N, g->K, tn);
    if (!g->A || !g->W || !g->C) FAIL(PMA_ERR_NULL, "A, W and C are required");
    if (g->lda < g->K || g->ldw < g->K || g->ldc < g->N)
        FAIL(PMA_ERR_SHAPE, "leading dimensions smaller than the matrix rows");
    if (g->lda % 8 || g->ldw % 8 || g->ldc % 8 || !aligned(g->A, 16) || !aligned(g->W, 16) ||
        !aligned(g->C, 16))
        FAIL(PMA_ERR_ALIGN, "A, W, C must be 16-byte aligned with leading dims %% 8 == 0");
    const int64_t wrows = g->epilogue == PMA_EPI_SWIGLU ? 2ll * g->N : g->N;
    if (!fits32(g->M, g->lda) || !fits32(wrows, g->ldw))
        FAIL(PMA_ERR_SHAPE, "A or W spans 2 GiB or more");
    if (g->epilogue == PMA_EPI_GATE_RESIDUAL) {
        if (!g->R || !g->table || !g->token_tags || !g->timestep_indices)
            FAIL(PMA_ERR_NULL, "gate-residual needs R, table, tags and timestep indices");
        if (g->ldr < g->N || g->ldr % 8 || !aligned(g->R, 16) || !aligned(g->table, 16))
            FAIL(PMA_ERR_ALIGN, "R / table alignment");
        if (g->num_timesteps < 1 || g->gate_chunk < 0 || g->gate_chunk > 5)
            FAIL(PMA_ERR_SHAPE, "num_timesteps %d gate_chunk %d", g->num_timesteps, g->gate_chunk);
    }
    pma_status st;
    if ((st = api_check_device()) != PMA_OK) return st;
    GemmLaunch a;
    memset(&a, 0, sizeof a);
    a.M = g->M; a.N = g->N; a.K = g->K;
    a.A = g->A; a.lda = g->lda;
    a.W = g->W; a.ldw = g->ldw;
    a.w_bytes = (uint32_t)(wrows * g->ldw * 2);
    a.C = g->C; a.ldc = g->ldc;
    a.epi = g->epilogue;
    a.R = g->R; a.ldr = g->ldr;
    a.table = g->table; a.T = g->num_timesteps; a.gate_chunk = g->gate_chunk;
    a.tags = g->token_tags; a.ts_idx = g->timestep_indices;
    if (stats) {
        a.epi = kEpiGateStats;
        a.stats = stats;
        a.stats_groups = stats_groups;
    }
    CHECK_HIP(launch_gemm(a, static_cast<hipStream_t>(stream)), "gemm launch");
    return PMA_OK;
}

}  // namespace

extern "C" {

pma_status pma_linear(const pma_linear_args *g, void *stream) { return linear_impl(g, nullptr, 0, stream); }

pma_status pma_gate_ln_workspace_size(const pma_block_params *p, int32_t seq_len, size_t *bytes) {
    pma_status st;
    if ((st = check_block_params(p)) != PMA_OK) return st;
    if (!bytes) FAIL(PMA_ERR_NULL, "bytes is NULL");
    if (seq_len < 1 || seq_len > (1 << 24)) FAIL(PMA_ERR_SHAPE, "seq_len %d", seq_len);
    // at most hidden / 128 groups per row (the narrower group width)
    *bytes = round_up((size_t)seq_len * (size_t)(p->hidden / 128) * sizeof(float2), 256);
    return PMA_OK;
}

pma_status pma_gate_residual_ln_modulate(const pma_block_params *p, const pma_layout *layout,
                                         const pma_bf16 *a_in, int64_t lda, int32_t K,
                                         const pma_bf16 *w, const float *gate_table,
                                         int32_t gate_chunk, const pma_bf16 *x, pma_bf16 *x1,
                                         const float *mod_table, int32_t which, pma_bf16 *b,
                                         void *workspace, size_t workspace_bytes, void *stream) {
    pma_status st;
    if ((st = check_block_params(p)) != PMA_OK) return st;
    if (!layout || !layout->token_tags || !layout->timestep_indices)
        FAIL(PMA_ERR_NULL, "layout is not built");
    if (!mod_table || !b || !workspace) FAIL(PMA_ERR_NULL, "mod_table, b and workspace are required");
    if (which != 0 && which != 1) FAIL(PMA_ERR_SHAPE, "which %d (0 or 1)", which);
    if (gate_chunk != 2 && gate_chunk != 5) FAIL(PMA_ERR_SHAPE, "gate_chunk %d (2 or 5)", gate_chunk);
    if (!aligned(b, 16) || !aligned(mod_table, 16) || !aligned(workspace, 256))
        FAIL(PMA_ERR_ALIGN, "b, mod_table 16-byte and workspace 256-byte aligned");
    const int32_t L = layout->seq_len, hid = p->hidden;
    size_t need = 0;
    if ((st = pma_gate_ln_workspace_size(p, L, &need)) != PMA_OK) return st;
    if (workspace_bytes < need) FAIL(PMA_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    const int gw = gemm_stats_group_width(L, hid);
    float2 *stats = static_cast<float2 *>(workspace);
    // x1 = x + gate (a w^T), rounded, with each row's statistics per group
    pma_linear_args g;
    memset(&g, 0, sizeof g);
    g.M = L; g.N = hid; g.K = K;
    g.A = a_in; g.lda = lda; g.W = w; g.ldw = K; g.C = x1; g.ldc = hid;
    g.epilogue = PMA_EPI_GATE_RESIDUAL;
    g.R = x; g.ldr = hid; g.table = gate_table; g.num_timesteps = layout->num_timesteps;
    g.gate_chunk = gate_chunk; g.token_tags = layout->token_tags;
    g.timestep_indices = layout->timestep_indices;
    if ((st = linear_impl(&g, stats, hid / gw, stream)) != PMA_OK) return st;
    // b = LN(x1) (1 + scale) + shift from those statistics
    LnModLaunch m;
    m.L = L;
    m.hidden = hid;
    m.T = layout->num_timesteps;
    m.shift_chunk = which ? 3 : 0;
    m.eps = p->norm_eps;
    m.x = x1;
    m.out = b;
    m.table = mod_table;
    m.tags = layout->token_tags;
    m.ts_idx = layout->timestep_indices;
    m.stats = stats;
    m.stats_groups = hid / gw;
    m.stats_gw = gw;
    CHECK_HIP(launch_ln_modulate(m, static_cast<hipStream_t>(stream)), "ln_modulate launch");
    return PMA_OK;
}

pma_status pma_rope_table(const pma_attn_params *p, const pma_layout *layout, float *table,
                          void *stream) {
    pma_status st;
    if ((st = api_check_attn_params(p)) != PMA_OK) return st;
    if ((st = api_check_layout(layout)) != PMA_OK) return st;
    if (!table) FAIL(PMA_ERR_NULL, "table is NULL");
    if (!aligned(table, 8)) FAIL(PMA_ERR_ALIGN, "table must be 8-byte aligned");
    if ((st = api_check_device()) != PMA_OK) return st;
    PrepLaunch a;
    memset(&a, 0, sizeof a);
    a.L = layout->seq_len;
    a.F = p->rope_freq_dim;
    api_fill_rope(p, a);
    a.pos = layout->position_ids;
    CHECK_HIP(launch_rope_table(a, reinterpret_cast<float2 *>(table), static_cast<hipStream_t>(stream)),
              "rope table launch");
    return PMA_OK;
}

pma_status pma_qkv_projection(const pma_attn_params *p, const pma_layout *layout,
                              const pma_bf16 *a_in, int64_t lda, int32_t hidden,
                              const pma_bf16 *w_qkv, const float *q_norm_weight,
                              const float *k_norm_weight, const float *rope_table,
                              pma_bf16 *qh, pma_bf16 *kh, pma_bf16 *vt, void *stream) {
    pma_status st;
    if ((st = api_check_attn_params(p)) != PMA_OK) return st;
    if ((st = api_check_layout(layout)) != PMA_OK) return st;
    const int32_t H = p->num_heads, L = layout->seq_len;
    if (H % 2 != 0) FAIL(PMA_ERR_SHAPE, "num_heads %d: the fused projection needs an even count", H);
    if (hidden < 64 || hidden % 64 != 0) FAIL(PMA_ERR_SHAPE, "hidden %d (multiple of 64)", hidden);
    if (!a_in || !w_qkv || !q_norm_weight || !k_norm_weight || !rope_table || !qh || !kh || !vt)
        FAIL(PMA_ERR_NULL, "a, w_qkv, norm weights, rope table and outputs are required");
    if (lda < hidden || lda % 8 != 0) FAIL(PMA_ERR_SHAPE, "lda %lld", (long long)lda);
    if (!aligned(a_in, 16) || !aligned(w_qkv, 16) || !aligned(qh, 16) || !aligned(kh, 16) ||
        !aligned(vt, 16) || !aligned(rope_table, 16) || !aligned(q_norm_weight, 16) ||
        !aligned(k_norm_weight, 16))
        FAIL(PMA_ERR_ALIGN, "a, w_qkv, qh, kh, vt, rope table and norm weights 16-byte aligned");
    const int64_t HD = (int64_t)H * kHeadDim;
    if (!fits32(L, lda) || !fits32(3 * HD, hidden)) FAIL(PMA_ERR_SHAPE, "A or W spans 2 GiB or more");
    if ((st = api_check_device()) != PMA_OK) return st;
    GemmLaunch g;
    memset(&g, 0, sizeof g);
    g.M = L; g.N = (int32_t)(3 * HD); g.K = hidden;
    g.A = a_in; g.lda = lda;
    g.W = w_qkv; g.ldw = hidden;
    g.w_bytes = (uint32_t)(3 * HD * hidden * 2);
    g.epi = p->rope_freq_dim == 16 ? kEpiQkvRope : kEpiQkvRope + 1;
    g.Lp = api_padded_len(L); g.H = H; g.F = p->rope_freq_dim;
    g.eps = p->qk_norm_eps;
    g.qscale = api_q_operand_scale(p);
    g.wq = q_norm_weight; g.wk = k_norm_weight;
    g.rope = reinterpret_cast<const float2 *>(rope_table);
    g.qh = qh; g.kh = kh; g.vt = vt;
    CHECK_HIP(launch_gemm(g, static_cast<hipStream_t>(stream)), "qkv projection launch");
    return PMA_OK;
}

// Workspace: a|b [L][hidden] | x1 [L][hidden] | h [L][ffn] | o [L][HD]
//            | attention operands (qh, kh, vt) | rope table [L][3F] float2
pma_status pma_block_workspace_size(const pma_block_params *p, int32_t L, size_t *bytes) {
    pma_status st;
    if ((st = check_block_params(p)) != PMA_OK) return st;
    if (!bytes) FAIL(PMA_ERR_NULL, "bytes is NULL");
    if (L < 1 || L > (1 << 24)) FAIL(PMA_ERR_SHAPE, "seq_len %d", L);
    const size_t HD = (size_t)p->attn.num_heads * kHeadDim;
    const size_t wide = (size_t)p->ffn_dim;
    size_t attn = 0;
    if ((st = pma_attention_workspace_size(&p->attn, L, &attn)) != PMA_OK) return st;
    *bytes = round_up((size_t)L * p->hidden * 2, 256) * 2 + round_up((size_t)L * wide * 2, 256) +
             round_up((size_t)L * HD * 2, 256) + attn +
             round_up((size_t)L * 3 * p->attn.rope_freq_dim * 8, 256);
    return PMA_OK;
}

}  // extern "C"

namespace {

// One block; rope_ready: the workspace's RoPE table already holds this
// layout's cos/sin (the stack builds it once for all its blocks).
pma_status block_forward_impl(const pma_block_params *p, const pma_layout *layout,
                              const pma_block_weights *w, const float *table,
                              const pma_bf16 *x_in, pma_bf16 *x_out, void *workspace,
                              size_t workspace_bytes, bool rope_ready, void *stream) {
    pma_status st;
    if ((st = check_block_params(p)) != PMA_OK) return st;
    if (!layout || !w || !table || !x_in || !x_out || !workspace)
        FAIL(PMA_ERR_NULL, "layout, weights, table, x_in, x_out and workspace are required");
    if (x_in == x_out) FAIL(PMA_ERR_SHAPE, "x_out must not alias x_in");
    if (!w->w_qkv || !w->w_o || !w->w_fc1 || !w->w_fc2 || !w->q_norm_weight || !w->k_norm_weight)
        FAIL(PMA_ERR_NULL, "a block weight is NULL");
    const int32_t L = layout->seq_len;
    size_t need = 0;
    if ((st = pma_block_workspace_size(p, L, &need)) != PMA_OK) return st;
    if (workspace_bytes < need)
        FAIL(PMA_ERR_WORKSPACE, "block workspace %zu < %zu bytes", workspace_bytes, need);
    if (!aligned(workspace, 256)) FAIL(PMA_ERR_ALIGN, "workspace must be 256-byte aligned");

    const int32_t hid = p->hidden, H = p->attn.num_heads, ffn = p->ffn_dim;
    const int64_t HD = (int64_t)H * kHeadDim;
    char *ws = static_cast<char *>(workspace);
    pma_bf16 *ab = reinterpret_cast<pma_bf16 *>(ws);                       // a, then b
    ws += round_up((size_t)L * hid * 2, 256);
    pma_bf16 *x1 = reinterpret_cast<pma_bf16 *>(ws);
    ws += round_up((size_t)L * hid * 2, 256);
    pma_bf16 *h = reinterpret_cast<pma_bf16 *>(ws);
    ws += round_up((size_t)L * ffn * 2, 256);
    pma_bf16 *o = reinterpret_cast<pma_bf16 *>(ws);
    ws += round_up((size_t)L * HD * 2, 256);
    void *attn_ws = ws;
    size_t attn_bytes = 0;
    if ((st = pma_attention_workspace_size(&p->attn, L, &attn_bytes)) != PMA_OK) return st;
    ws += attn_bytes;
    float *rope = reinterpret_cast<float *>(ws);

    // a = LN(x) (1 + scale_a) + shift_a
    if ((st = pma_ln_modulate(p, layout, table, 0, x_in, ab, stream)) != PMA_OK) return st;
    // Q', K' (normed, rotated) and V^T straight from the QKV projection
    const int32_t Lp = api_padded_len(L);
    const size_t one = round_up((size_t)H * Lp * kHeadDim * 2, 256);
    pma_bf16 *qh = static_cast<pma_bf16 *>(attn_ws);
    pma_bf16 *kh = reinterpret_cast<pma_bf16 *>(static_cast<char *>(attn_ws) + one);
    pma_bf16 *vt = reinterpret_cast<pma_bf16 *>(static_cast<char *>(attn_ws) + 2 * one);
    if (!rope_ready && (st = pma_rope_table(&p->attn, layout, rope, stream)) != PMA_OK) return st;
    if ((st = pma_qkv_projection(&p->attn, layout, ab, hid, hid, w->w_qkv, w->q_norm_weight,
                                 w->k_norm_weight, rope, qh, kh, vt, stream)) != PMA_OK)
        return st;
    if ((st = pma_flash_attention(&p->attn, layout, qh, kh, vt, o, HD, nullptr,
                                  static_cast<char *>(attn_ws) + 3 * one, attn_bytes - 3 * one,
                                  stream)) != PMA_OK)
        return st;
    pma_linear_args g;
    // x1 = x + gate_a (O W_o^T).  (pma_gate_residual_ln_modulate would take
    // x1's row statistics in this epilogue for the norm below; measured at
    // L = 8192 it is 0.8% slower than the two launches: the norm pass already
    // streams at the device-copy rate, and the statistics cost the epilogue.)
    memset(&g, 0, sizeof g);
    g.M = L; g.N = hid; g.K = (int32_t)HD;
    g.A = o; g.lda = HD; g.W = w->w_o; g.ldw = HD; g.C = x1; g.ldc = hid;
    g.epilogue = PMA_EPI_GATE_RESIDUAL;
    g.R = x_in; g.ldr = hid; g.table = table; g.num_timesteps = layout->num_timesteps;
    g.gate_chunk = 2; g.token_tags = layout->token_tags; g.timestep_indices = layout->timestep_indices;
    if ((st = pma_linear(&g, stream)) != PMA_OK) return st;
    // b = LN(x1) (1 + scale_f) + shift_f
    if ((st = pma_ln_modulate(p, layout, table, 1, x1, ab, stream)) != PMA_OK) return st;
    // h = silu(b W_gate^T) (b W_up^T)
    memset(&g, 0, sizeof g);
    g.M = L; g.N = ffn; g.K = hid;
    g.A = ab; g.lda = hid; g.W = w->w_fc1; g.ldw = hid; g.C = h; g.ldc = ffn;
    g.epilogue = PMA_EPI_SWIGLU;
    if ((st = pma_linear(&g, stream)) != PMA_OK) return st;
    // x2 = x1 + gate_f (h W_fc2^T)
    memset(&g, 0, sizeof g);
    g.M = L; g.N = hid; g.K = ffn;
    g.A = h; g.lda = ffn; g.W = w->w_fc2; g.ldw = ffn; g.C = x_out; g.ldc = hid;
    g.epilogue = PMA_EPI_GATE_RESIDUAL;
    g.R = x1; g.ldr = hid; g.table = table; g.num_timesteps = layout->num_timesteps;
    g.gate_chunk = 5; g.token_tags = layout->token_tags; g.timestep_indices = layout->timestep_indices;
    return pma_linear(&g, stream);
}

// Byte offset of the RoPE table inside a block workspace.
size_t block_rope_offset(const pma_block_params *p, int32_t L) {
    const size_t HD = (size_t)p->attn.num_heads * kHeadDim;
    size_t attn = 0;
    pma_attention_workspace_size(&p->attn, L, &attn);
    return round_up((size_t)L * p->hidden * 2, 256) * 2 + round_up((size_t)L * p->ffn_dim * 2, 256) +
           round_up((size_t)L * HD * 2, 256) + attn;
}

size_t table_bytes(const pma_block_params *p, int32_t T) {
    return round_up((size_t)3 * T * 6 * p->hidden * 4, 256);
}

}  // namespace

extern "C" {

pma_status pma_block_forward(const pma_block_params *p, const pma_layout *layout,
                             const pma_block_weights *w, const float *table,
                             const pma_bf16 *x_in, pma_bf16 *x_out, void *workspace,
                             size_t workspace_bytes, void *stream) {
    return block_forward_impl(p, layout, w, table, x_in, x_out, workspace, workspace_bytes, false,
                              stream);
}

// Stack workspace: block workspace | AdaLN table [3][T][6][hidden] fp32 | x [L][hidden] bf16
pma_status pma_stack_workspace_size(const pma_block_params *p, int32_t L, int32_t T,
                                    size_t *bytes) {
    pma_status st;
    size_t blk = 0;
    if ((st = pma_block_workspace_size(p, L, &blk)) != PMA_OK) return st;
    if (T < 1 || T > adaln_max_t()) FAIL(PMA_ERR_SHAPE, "num_timesteps %d (1..%d)", T, adaln_max_t());
    *bytes = blk + table_bytes(p, T) + round_up((size_t)L * p->hidden * 2, 256);
    return PMA_OK;
}

pma_status pma_stack_forward(const pma_block_params *p, const pma_layout *layout,
                             int32_t num_blocks, const pma_block_weights *w,
                             const pma_bf16 *temb, const pma_bf16 *x_in, pma_bf16 *x_out,
                             void *workspace, size_t workspace_bytes, void *stream) {
    pma_status st;
    if ((st = check_block_params(p)) != PMA_OK) return st;
    if ((st = api_check_layout(layout)) != PMA_OK) return st;
    if (num_blocks < 1) FAIL(PMA_ERR_SHAPE, "num_blocks %d", num_blocks);
    if (!w || !temb || !x_in || !x_out || !workspace)
        FAIL(PMA_ERR_NULL, "weights, temb, x_in, x_out and workspace are required");
    if (x_in == x_out) FAIL(PMA_ERR_SHAPE, "x_out must not alias x_in");
    for (int32_t l = 0; l < num_blocks; ++l)
        if (!w[l].w_ada || !w[l].w_qkv || !w[l].w_o || !w[l].w_fc1 || !w[l].w_fc2 ||
            !w[l].q_norm_weight || !w[l].k_norm_weight)
            FAIL(PMA_ERR_NULL, "a weight of block %d is NULL", l);
    const int32_t L = layout->seq_len, T = layout->num_timesteps;
    size_t need = 0, blk = 0;
    if ((st = pma_stack_workspace_size(p, L, T, &need)) != PMA_OK) return st;
    if ((st = pma_block_workspace_size(p, L, &blk)) != PMA_OK) return st;
    if (workspace_bytes < need)
        FAIL(PMA_ERR_WORKSPACE, "stack workspace %zu < %zu bytes", workspace_bytes, need);
    if (!aligned(workspace, 256)) FAIL(PMA_ERR_ALIGN, "workspace must be 256-byte aligned");
    char *ws = static_cast<char *>(workspace);
    float *table = reinterpret_cast<float *>(ws + blk);
    pma_bf16 *tmp = reinterpret_cast<pma_bf16 *>(ws + blk + table_bytes(p, T));
    // the RoPE table depends only on the layout: built once for every block
    float *rope = reinterpret_cast<float *>(ws + block_rope_offset(p, L));
    if ((st = pma_rope_table(&p->attn, layout, rope, stream)) != PMA_OK) return st;
    // block l writes x_out when (num_blocks - 1 - l) is even, tmp otherwise,
    // so the last block lands in x_out and no block reads what it writes
    const pma_bf16 *src = x_in;
    for (int32_t l = 0; l < num_blocks; ++l) {
        pma_bf16 *dst = ((num_blocks - 1 - l) % 2 == 0) ? x_out : tmp;
        if ((st = pma_adaln_table(p, T, temb, w[l].w_ada, table, stream)) != PMA_OK) return st;
        if ((st = block_forward_impl(p, layout, &w[l], table, src, dst, workspace, blk, true,
                                     stream)) != PMA_OK)
            return st;
        src = dst;
    }
    return PMA_OK;
}

pma_status pma_token_merge(int32_t hidden, int32_t seq_len, int32_t n_reduced,
                           const int32_t *src0, const int32_t *src1, const pma_bf16 *x,
                           pma_bf16 *xr, void *stream) {
    if (hidden < 8 || hidden % 8 != 0) FAIL(PMA_ERR_SHAPE, "hidden %d (multiple of 8)", hidden);
    if (seq_len < 1 || n_reduced < 0 || n_reduced > seq_len)
        FAIL(PMA_ERR_SHAPE, "seq_len %d, n_reduced %d", seq_len, n_reduced);
    if (n_reduced && (!src0 || !src1 || !x || !xr)) FAIL(PMA_ERR_NULL, "src0, src1, x and xr are required");
    if (!aligned(x, 16) || !aligned(xr, 16)) FAIL(PMA_ERR_ALIGN, "x and xr must be 16-byte aligned");
    pma_status st;
    if ((st = api_check_device()) != PMA_OK) return st;
    TokenLaunch a;
    memset(&a, 0, sizeof a);
    a.n = n_reduced; a.hidden = hidden; a.L = seq_len;
    a.src0 = src0; a.src1 = src1; a.x = x; a.xr_out = xr;
    CHECK_HIP(launch_token_merge(a, static_cast<hipStream_t>(stream)), "token merge launch");
    return PMA_OK;
}

pma_status pma_token_restore(int32_t hidden, int32_t seq_len, int32_t n_reduced,
                             const int32_t *src0, const int32_t *src1, const pma_bf16 *bypass,
                             const pma_bf16 *xr_before, const pma_bf16 *xr_after,
                             pma_bf16 *x_out, void *stream) {
    if (hidden < 8 || hidden % 8 != 0) FAIL(PMA_ERR_SHAPE, "hidden %d (multiple of 8)", hidden);
    if (seq_len < 1 || n_reduced < 0 || n_reduced > seq_len)
        FAIL(PMA_ERR_SHAPE, "seq_len %d, n_reduced %d", seq_len, n_reduced);
    if (n_reduced && (!src0 || !src1 || !bypass || !xr_before || !xr_after || !x_out))
        FAIL(PMA_ERR_NULL, "src0, src1, bypass, xr_before, xr_after and x_out are required");
    if (!aligned(bypass, 16) || !aligned(xr_before, 16) || !aligned(xr_after, 16) || !aligned(x_out, 16))
        FAIL(PMA_ERR_ALIGN, "row arrays must be 16-byte aligned");
    pma_status st;
    if ((st = api_check_device()) != PMA_OK) return st;
    TokenLaunch a;
    memset(&a, 0, sizeof a);
    a.n = n_reduced; a.hidden = hidden; a.L = seq_len;
    a.src0 = src0; a.src1 = src1; a.x = bypass; a.xr_before = xr_before; a.xr_in = xr_after;
    a.x_out = x_out;
    CHECK_HIP(launch_token_restore(a, static_cast<hipStream_t>(stream)), "token restore launch");
    return PMA_OK;
}

pma_status pma_token_plan_check(int32_t seq_len, int32_t n_reduced, const int32_t *src0,
                                const int32_t *src1, int32_t *workspace, void *stream,
                                int32_t *bits, int32_t *first_bad_entry, int32_t *first_bad_row) {
    if (seq_len < 1 || n_reduced < 0 || n_reduced > seq_len)
        FAIL(PMA_ERR_SHAPE, "seq_len %d, n_reduced %d", seq_len, n_reduced);
    if ((n_reduced && (!src0 || !src1)) || !workspace)
        FAIL(PMA_ERR_NULL, "src0, src1 and workspace are required");
    if (!aligned(workspace, 4)) FAIL(PMA_ERR_ALIGN, "workspace must be 4-byte aligned");
    pma_status st;
    if ((st = api_check_device()) != PMA_OK) return st;
    TokenLaunch a;
    memset(&a, 0, sizeof a);
    a.n = n_reduced; a.L = seq_len; a.src0 = src0; a.src1 = src1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    CHECK_HIP(launch_token_plan_check(a, workspace, s), "token plan check launch");
    int32_t h[3] = {0, 0, 0};
    CHECK_HIP(hipMemcpyAsync(h, workspace, sizeof h, hipMemcpyDeviceToHost, s), "plan status copy");
    CHECK_HIP(hipStreamSynchronize(s), "plan status sync");
    const int32_t fe = h[1] == 0x7fffffff ? -1 : h[1], fr = h[2] == 0x7fffffff ? -1 : h[2];
    if (bits) *bits = h[0];
    if (first_bad_entry) *first_bad_entry = fe;
    if (first_bad_row) *first_bad_row = fr;
    if (h[0] != 0)
        FAIL(PMA_ERR_LAYOUT, "token plan status bits 0x%x, first bad entry %d, first bad row %d", h[0],
             fe, fr);
    return PMA_OK;
}

// Refiner workspace: projected text [n][hidden] bf16 | stack workspace
pma_status pma_refiner_workspace_size(const pma_block_params *p, int32_t n, int32_t T,
                                      size_t *bytes) {
    pma_status st;
    size_t stack = 0;
    if ((st = pma_stack_workspace_size(p, n, T, &stack)) != PMA_OK) return st;
    *bytes = round_up((size_t)n * p->hidden * 2, 256) + stack;
    return PMA_OK;
}

pma_status pma_text_refiner(const pma_block_params *p, const pma_layout *text_layout,
                            int32_t num_blocks, const pma_block_weights *w,
                            const pma_bf16 *temb, const pma_bf16 *text, int64_t text_ld,
                            int32_t text_dim, const pma_bf16 *w_text, float final_norm_eps,
                            pma_bf16 *out, void *workspace, size_t workspace_bytes,
                            void *stream) {
    pma_status st;
    if ((st = check_block_params(p)) != PMA_OK) return st;
    if ((st = api_check_layout(text_layout)) != PMA_OK) return st;
    if (num_blocks < 0) FAIL(PMA_ERR_SHAPE, "num_blocks %d", num_blocks);
    if (!text || !w_text || !out || !workspace) FAIL(PMA_ERR_NULL, "text, w_text, out and workspace are required");
    if (num_blocks > 0 && (!w || !temb)) FAIL(PMA_ERR_NULL, "block weights and temb are required");
    if (text_dim < 64 || text_dim % 64 != 0 || text_ld < text_dim || text_ld % 8 != 0)
        FAIL(PMA_ERR_SHAPE, "text_dim %d (multiple of 64), text_ld %lld", text_dim, (long long)text_ld);
    if (!(final_norm_eps >= 0.f)) FAIL(PMA_ERR_SHAPE, "final_norm_eps %g", (double)final_norm_eps);
    if (!aligned(text, 16) || !aligned(w_text, 16) || !aligned(out, 16))
        FAIL(PMA_ERR_ALIGN, "text, w_text and out must be 16-byte aligned");
    const int32_t n = text_layout->seq_len, T = text_layout->num_timesteps;
    size_t need = 0;
    if ((st = pma_refiner_workspace_size(p, n, T, &need)) != PMA_OK) return st;
    if (workspace_bytes < need)
        FAIL(PMA_ERR_WORKSPACE, "refiner workspace %zu < %zu bytes", workspace_bytes, need);
    if (!aligned(workspace, 256)) FAIL(PMA_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (!fits32(n, text_ld) || !fits32(p->hidden, text_dim)) FAIL(PMA_ERR_SHAPE, "text spans 2 GiB or more");
    char *ws = static_cast<char *>(workspace);
    pma_bf16 *proj = reinterpret_cast<pma_bf16 *>(ws);
    const size_t proj_bytes = round_up((size_t)n * p->hidden * 2, 256);
    // text projection (bf16 stack, no bias)
    pma_linear_args g;
    memset(&g, 0, sizeof g);
    g.M = n; g.N = p->hidden; g.K = text_dim;
    g.A = text; g.lda = text_ld; g.W = w_text; g.ldw = text_dim; g.C = proj; g.ldc = p->hidden;
    g.epilogue = PMA_EPI_STORE;
    if ((st = pma_linear(&g, stream)) != PMA_OK) return st;
    const pma_bf16 *last = proj;
    if (num_blocks > 0) {
        if ((st = pma_stack_forward(p, text_layout, num_blocks, w, temb, proj, out, ws + proj_bytes,
                                    workspace_bytes - proj_bytes, stream)) != PMA_OK)
            return st;
        last = out;
    }
    // output norm: LayerNorm without modulation, eps = final_norm_eps (in place when
    // the blocks already wrote out)
    LnModLaunch a;
    memset(&a, 0, sizeof a);
    a.L = n;
    a.hidden = p->hidden;
    a.T = T;
    a.eps = final_norm_eps;
    a.x = last;
    a.out = out;
    a.table = nullptr;
    a.tags = text_layout->token_tags;
    a.ts_idx = text_layout->timestep_indices;
    CHECK_HIP(launch_ln_modulate(a, static_cast<hipStream_t>(stream)), "refiner norm launch");
    return PMA_OK;
}

}  // extern "C"
