// block_api.cpp -- C ABI of the DiT block pieces: argument checks and launches.
// The operations and their page citations are documented in include/pma.h.
#include <hip/hip_runtime.h>

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
    CHECK_HIP(launch_ln_modulate(a, static_cast<hipStream_t>(stream)), "ln_modulate launch");
    return PMA_OK;
}

pma_status pma_linear(const pma_linear_args *g, void *stream) {
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
    CHECK_HIP(launch_gemm(a, static_cast<hipStream_t>(stream)), "gemm launch");
    return PMA_OK;
}

// Workspace: a|b [L][hidden] | qkv|h [L][max(3HD, ffn)] | o [L][HD] | x1 [L][hidden]
//            | attention operands (qh, kh, vt)
pma_status pma_block_workspace_size(const pma_block_params *p, int32_t L, size_t *bytes) {
    pma_status st;
    if ((st = check_block_params(p)) != PMA_OK) return st;
    if (!bytes) FAIL(PMA_ERR_NULL, "bytes is NULL");
    if (L < 1 || L > (1 << 24)) FAIL(PMA_ERR_SHAPE, "seq_len %d", L);
    const size_t HD = (size_t)p->attn.num_heads * kHeadDim;
    const size_t wide = HD * 3 > (size_t)p->ffn_dim ? HD * 3 : (size_t)p->ffn_dim;
    size_t attn = 0;
    if ((st = pma_attention_workspace_size(&p->attn, L, &attn)) != PMA_OK) return st;
    *bytes = round_up((size_t)L * p->hidden * 2, 256) * 2 + round_up((size_t)L * wide * 2, 256) +
             round_up((size_t)L * HD * 2, 256) + attn;
    return PMA_OK;
}

pma_status pma_block_forward(const pma_block_params *p, const pma_layout *layout,
                             const pma_block_weights *w, const float *table,
                             const pma_bf16 *x_in, pma_bf16 *x_out, void *workspace,
                             size_t workspace_bytes, void *stream) {
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
    const int64_t wide = HD * 3 > ffn ? HD * 3 : ffn;
    char *ws = static_cast<char *>(workspace);
    pma_bf16 *ab = reinterpret_cast<pma_bf16 *>(ws);                       // a, then b
    ws += round_up((size_t)L * hid * 2, 256);
    pma_bf16 *x1 = reinterpret_cast<pma_bf16 *>(ws);
    ws += round_up((size_t)L * hid * 2, 256);
    pma_bf16 *qkvh = reinterpret_cast<pma_bf16 *>(ws);                     // qkv, then h
    ws += round_up((size_t)L * wide * 2, 256);
    pma_bf16 *o = reinterpret_cast<pma_bf16 *>(ws);
    ws += round_up((size_t)L * HD * 2, 256);
    void *attn_ws = ws;
    const size_t attn_bytes = workspace_bytes - (size_t)(ws - static_cast<char *>(workspace));

    // a = LN(x) (1 + scale_a) + shift_a
    if ((st = pma_ln_modulate(p, layout, table, 0, x_in, ab, stream)) != PMA_OK) return st;
    // [Q|K|V] = a W_qkv^T
    pma_linear_args g;
    memset(&g, 0, sizeof g);
    g.M = L; g.N = (int32_t)(3 * HD); g.K = hid;
    g.A = ab; g.lda = hid; g.W = w->w_qkv; g.ldw = hid; g.C = qkvh; g.ldc = 3 * HD;
    g.epilogue = PMA_EPI_STORE;
    if ((st = pma_linear(&g, stream)) != PMA_OK) return st;
    // attention path on the token-major Q, K, V columns
    if ((st = pma_attention(&p->attn, layout, qkvh, 3 * HD, qkvh + HD, 3 * HD, qkvh + 2 * HD,
                            3 * HD, w->q_norm_weight, w->k_norm_weight, o, HD, nullptr, attn_ws,
                            attn_bytes, stream)) != PMA_OK)
        return st;
    // x1 = x + gate_a (O W_o^T)
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
    g.A = ab; g.lda = hid; g.W = w->w_fc1; g.ldw = hid; g.C = qkvh; g.ldc = ffn;
    g.epilogue = PMA_EPI_SWIGLU;
    if ((st = pma_linear(&g, stream)) != PMA_OK) return st;
    // x2 = x1 + gate_f (h W_fc2^T)
    memset(&g, 0, sizeof g);
    g.M = L; g.N = hid; g.K = ffn;
    g.A = qkvh; g.lda = ffn; g.W = w->w_fc2; g.ldw = ffn; g.C = x_out; g.ldc = hid;
    g.epilogue = PMA_EPI_GATE_RESIDUAL;
    g.R = x1; g.ldr = hid; g.table = table; g.num_timesteps = layout->num_timesteps;
    g.gate_chunk = 5; g.token_tags = layout->token_tags; g.timestep_indices = layout->timestep_indices;
    return pma_linear(&g, stream);
}

}  // extern "C"
