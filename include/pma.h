/*
 * pma.h -- C ABI of libpma: packed masked attention and the MiniMax-H3 DiT
 * block on AMD Instinct MI355X (gfx950).
 *
 * Every entry point takes plain pointers and sizes.  Unless stated otherwise
 * a pointer argument is a DEVICE pointer owned by the caller; the library
 * never allocates or frees device memory and keeps no state between calls
 * beyond a per-thread error string and a per-device property cache.  Kernels
 * are launched asynchronously on `stream` (a hipStream_t; NULL = the default
 * stream); a call returns once its kernels are queued.  Calls on different
 * streams are independent.  No C++ exception crosses this interface.
 *
 * Errors: argument checks that need no device data run on the host before any
 * launch and return a status without launching anything.  Checks that depend
 * on device data (the packed layout's contents) are done by a kernel that
 * writes a status word into the layout workspace; pma_layout_read_status()
 * reads it back.  HIP runtime failures return PMA_ERR_DEVICE.  On every
 * non-OK return, pma_last_error() gives a human-readable detail string for
 * the calling thread.
 *
 * Pages cited (by title and section):
 *   [H3]  "MiniMaxH3Transformer3DModel" -- diffusers API page: intro,
 *         constructor parameters, class description, forward parameters.
 *   [ENG] "MiniMax H3 Inference Engine voor Mac computers" -- implementation
 *         notes ("Exacte DiT fusions", "Metal 4 en TensorOps pads",
 *         "Checkpoint layout en media pipeline", "Scheduling en
 *         activatiegeheugen").
 *
 * Storage types: bf16 tensors are passed as pma_bf16 (the raw 16-bit
 * pattern); every fp32 -> bf16 store rounds to nearest, ties to even.
 */
#ifndef PMA_H_
#define PMA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t pma_bf16; /* bfloat16 bit pattern */

typedef enum {
    PMA_OK = 0,
    PMA_ERR_NULL = 1,        /* a required pointer is NULL                     */
    PMA_ERR_SHAPE = 2,       /* a size, count or parameter is out of range     */
    PMA_ERR_ALIGN = 3,       /* a pointer or leading dimension is misaligned   */
    PMA_ERR_WORKSPACE = 4,   /* the workspace is smaller than required         */
    PMA_ERR_LAYOUT = 5,      /* the packed layout failed validation            */
    PMA_ERR_DEVICE = 6,      /* a HIP runtime call failed                      */
    PMA_ERR_UNSUPPORTED = 7  /* device is not gfx950, or unsupported option    */
} pma_status;

/* Static name of a status code. */
const char *pma_status_string(pma_status s);
/* Detail of the calling thread's last failed call ("" if none). */
const char *pma_last_error(void);
/* PMA_OK if the current HIP device is a gfx950; PMA_ERR_UNSUPPORTED if not. */
pma_status pma_device_check(void);

/* ======================================================================
 * 1. Packed layout -> documents and tile map
 * ----------------------------------------------------------------------
 * [H3] forward parameters: one packed 1-D sequence of L rows described by
 * token_tags (0 video, 1 text, 2 audio), position_ids (t, h, w) per row,
 * timestep_indices per row into T distinct timesteps, and three index
 * tensors with the positions of the video, audio and text rows.  [H3] intro:
 * rows tagged -1 are padding and form their own attention document through
 * a boolean mask; [H3] class description: the original reference splits the
 * padded tail off as its own varlen document.
 *
 * Document rule: row i may attend to row j iff (tag_i == -1) == (tag_j == -1).
 * All padding rows are one document, all other rows the other one.
 * ====================================================================== */

/* Layout status bits (OR-ed into the status word by pma_layout_build). */
#define PMA_LAYOUT_BAD_TAG        (1 << 0) /* tag not in {-1, 0, 1, 2}                 */
#define PMA_LAYOUT_BAD_TIMESTEP   (1 << 1) /* non-padding row, index outside [0, T)    */
#define PMA_LAYOUT_BAD_POSITION   (1 << 2) /* a position with |p| >= 2^24               */
#define PMA_LAYOUT_BAD_INDEX      (1 << 3) /* index tensor entry outside [0, L)         */
#define PMA_LAYOUT_UNSORTED_INDEX (1 << 4) /* index tensor not strictly ascending       */
#define PMA_LAYOUT_INDEX_TAG      (1 << 5) /* index names a row of another modality     */
#define PMA_LAYOUT_INDEX_COUNT    (1 << 6) /* count != number of rows with that tag     */

/* Tile classes of the (tile_m x tile_n) tiling of the L x L mask, over the
 * in-range pairs of each tile. */
#define PMA_TILE_EMPTY   0 /* no allowed pair: never visited   */
#define PMA_TILE_PARTIAL 1 /* some pairs allowed: masked tile  */
#define PMA_TILE_FULL    2 /* every in-range pair allowed      */

typedef struct {
    int32_t seq_len;                  /* L >= 1                                      */
    int32_t num_timesteps;            /* T >= 1                                      */
    const int32_t *token_tags;        /* [L]                                         */
    const int32_t *position_ids;      /* [L][3]  (t, h, w)                           */
    const int32_t *timestep_indices;  /* [L]     ignored on padding rows             */
    const int32_t *video_indices;     /* [num_video] ascending (NULL iff count 0)    */
    const int32_t *audio_indices;     /* [num_audio]                                 */
    const int32_t *text_indices;      /* [num_text]                                  */
    int32_t num_video, num_audio, num_text;
} pma_layout_desc;

/* A built layout: plain data, device pointers into the caller's workspace
 * plus copies of the descriptor's pointers.  Valid while the workspace and
 * the descriptor's arrays are. */
typedef struct {
    int32_t seq_len, num_timesteps;
    int32_t tile_m, tile_n;           /* tiling of the tile map                       */
    int32_t num_q_tiles, num_k_tiles; /* ceil(L / tile_m), ceil(L / tile_n)           */
    const int32_t *token_tags, *position_ids, *timestep_indices;
    int32_t *doc;                     /* [L]  1 for padding rows, 0 otherwise          */
    uint8_t *tile_class;              /* [num_q_tiles][num_k_tiles] PMA_TILE_*         */
    int32_t *tile_count;              /* [num_q_tiles] non-EMPTY k-tiles per q-tile    */
    int32_t *tile_list;               /* [num_q_tiles][num_k_tiles] ascending non-EMPTY
                                         k-tiles, then -1                              */
    int32_t *tile_order;              /* [num_q_tiles] q-tiles by (count desc, index asc) */
    int32_t *status;                  /* [2] status bits, first row with a per-row error
                                         (bad tag, timestep or position) or -1          */
    int32_t *scratch;                 /* builder's internal counters                  */
} pma_layout;

/* Bytes of device workspace pma_layout_build needs. */
pma_status pma_layout_workspace_size(int32_t seq_len, int32_t tile_m, int32_t tile_n,
                                     size_t *bytes);

/* Validate the layout and build document ids and the tile map.  tile_m and
 * tile_n must each be 64, 128 or 256 (pass 0, 0 for the attention kernel's
 * own tiling, see pma_attention_tiles).  workspace: >= the size above,
 * 256-byte aligned.  Writes *out on the host; the device arrays are ready
 * when the queued kernels finish.  The status word never makes a launch
 * fail: read it with pma_layout_read_status. */
pma_status pma_layout_build(const pma_layout_desc *desc, int32_t tile_m, int32_t tile_n,
                            void *workspace, size_t workspace_bytes, void *stream,
                            pma_layout *out);

/* Synchronise `stream` and copy the status word to the host.  Returns
 * PMA_ERR_LAYOUT if any status bit is set (PMA_OK otherwise); bits and
 * first_bad_row may be NULL. */
pma_status pma_layout_read_status(const pma_layout *layout, void *stream, int32_t *bits,
                                  int32_t *first_bad_row);

/* ======================================================================
 * 2. Attention path: QK-RMSNorm + 3-axis RoPE, masked flash attention
 * ----------------------------------------------------------------------
 * [H3] constructor parameters: num_attention_heads (56), attention_head_dim
 * (128), rope_freq_dim F (16): the t, h, w axes share one inv_freq buffer of
 * length F and 2*3*F of the head's channels are rotated; rope_theta (1e4);
 * qk_norm_eps (1e-5) of the per-head query/key norms.
 *
 * Computed, per row i and head h (readings of the pages' open points):
 *   n = x * w / sqrt(mean(x^2) + qk_norm_eps)        RMSNorm over the head's D
 *   axis a in {t,h,w}, f < F, phi = (pos[i][a] * pos_scale[a]) * theta^(-f/F),
 *   c0 = 2aF + f, c1 = c0 + F:
 *     y[c0] = n[c0] cos phi - n[c1] sin phi,  y[c1] = n[c1] cos phi + n[c0] sin phi
 *   y[c] = n[c] for c >= 6F.
 *   O_i = sum_{j in doc(i)} softmax_j(scale * q'_i . k'_j) v_j,  scale = 1/sqrt(D)
 * ====================================================================== */

typedef struct {
    int32_t num_heads;     /* H >= 1                                   */
    int32_t head_dim;      /* D; must be 128                           */
    int32_t rope_freq_dim; /* F; must be 8 or 16 (6F <= D)             */
    float rope_theta;      /* > 0                                      */
    float qk_norm_eps;     /* >= 0                                     */
    float softmax_scale;   /* 0 selects 1/sqrt(D)                      */
    float pos_scale[3];    /* per-axis scale of the (t, h, w) positions in
                              the rotation angle; 0 selects 1.  [ENG]
                              256x256 preview: the spatial coordinates are
                              halved (1, 0.5, 0.5) at the 8x8 token grid   */
} pma_attn_params;

/* The (tile_m, tile_n) the flash attention kernel needs its layout built with. */
pma_status pma_attention_tiles(int32_t *tile_m, int32_t *tile_n);

/* Padded row count Lp of the attention operands (L rounded up to 256). */
pma_status pma_attention_padded_len(int32_t seq_len, int32_t *padded_len);

/* QK-RMSNorm + 3-axis RoPE of Q and K, and relayout of Q, K, V into the
 * attention kernel's operands.
 *   q, k, v: token-major bf16, row i of head h at x[i*ld + h*D .. + D);
 *            ld >= H*D, ld % 8 == 0, 16-byte aligned (the QKV projection
 *            output [L][3*H*D] is used with ld = 3*H*D and offsets 0, HD, 2HD).
 *   q_norm_weight, k_norm_weight: fp32 [D], shared by all heads.
 *   qh, kh: bf16 [H][Lp][D] head-major normalised, rotated Q and K.  qh also
 *           carries the attention's logit factor: it holds the normalised,
 *           rotated Q times softmax_scale * log2(e) (both in fp32, rounded to
 *           bf16 once), so the attention kernel's QK product is the softmax
 *           exponent in base 2.
 *   vt:     bf16 [H][D][Lp] V transposed per head (keys contiguous).
 *   Rows L..Lp-1 of qh, kh and columns L..Lp-1 of vt are written as zero.
 * [ENG] "Checkpoint layout en media pipeline" fuses the QK norm with RoPE;
 * [ENG] "Metal 4 en TensorOps pads" feeds head-major attention inputs. */
pma_status pma_qk_norm_rope(const pma_attn_params *p, const pma_layout *layout,
                            const pma_bf16 *q, int64_t q_ld, const pma_bf16 *k,
                            int64_t k_ld, const pma_bf16 *v, int64_t v_ld,
                            const float *q_norm_weight, const float *k_norm_weight,
                            pma_bf16 *qh, pma_bf16 *kh, pma_bf16 *vt, void *stream);

/* Bytes of the optional workspace of pma_flash_attention: 256 bytes of
 * work-queue counters, then the partial results of the items whose key
 * ranges are split (none below 8192 keys), then (when any item is split)
 * 32 KiB of clock stamps: for each persistent workgroup of the last call
 * (at most 1024, one per CU), four u64 -- the shader clock counter and the
 * 100 MHz real-time counter at its start, the same two at its end -- from
 * which a caller can read the clock the kernel ran at. */
pma_status pma_flash_workspace_size(const pma_attn_params *p, int32_t seq_len, size_t *bytes);

/* Masked flash attention forward on the operands of pma_qk_norm_rope (or
 * pma_qkv_projection): the logit of query i and key j is qh[i].kh[j] in base
 * 2, i.e. the softmax scale is the one qh was produced with.
 * layout must be built with pma_attention_tiles()' tiling.  Tiles the layout
 * marks EMPTY are skipped whole; PARTIAL tiles and the ragged last k-tile
 * apply the document/bounds mask.
 *   o:   bf16 token-major, row i of head h at o[i*o_ld + h*D .. + D), o_ld >= H*D,
 *        o_ld % 8 == 0.  Only rows < L are written.
 *   lse: fp32 [H][L] natural-log sum of exp of the scaled logits (NULL: not written).
 *   workspace: NULL, or >= pma_flash_workspace_size() bytes, 256-byte aligned,
 *        owned by the caller and overwritten (contents need no clearing).
 *        From 8192 keys on, it holds a work queue: one workgroup per CU
 *        pulls (head, q-tile) items, first its own XCD's then what is left of
 *        the others', and the last items of every XCD's share run as two
 *        (below 12288 keys) or four parts over their key ranges, whose
 *        partial softmax results a second kernel merges.  Shorter sequences, or NULL, run one item per
 *        workgroup.  The two agree to fp32 rounding order (each part rounds
 *        its probabilities to bf16 against its own running maximum).
 *        Calls that share one workspace must not overlap.
 * The kernel keeps each q-tile's k-tile list in LDS: layouts of more than
 * 6908 k-tiles (seq_len > 442112) return PMA_ERR_SHAPE. */
pma_status pma_flash_attention(const pma_attn_params *p, const pma_layout *layout,
                               const pma_bf16 *qh, const pma_bf16 *kh, const pma_bf16 *vt,
                               pma_bf16 *o, int64_t o_ld, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Allocation-free form of pma_flash_attention, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks and results
 * contract as pma_flash_attention, without the workspace: the work-queue
 * counters and the split items' partial results live in a file-scope device
 * array of PMA_FLASH_STATIC_SCRATCH_BYTES (32 MiB) that every GPU the library
 * runs on holds until the process ends.  The array bounds the key-range
 * split to the items it holds: up to 7 split items per XCD (the workspace
 * form takes up to 16), so from 8192 keys on the two forms agree to fp32
 * rounding order, and below that bit for bit.  No shape is refused for the
 * array's size.  The call allocates nothing; the counters are cleared by a
 * kernel on the stream at every call.  All calls on one GPU share its array:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * not be issued. */
#define PMA_FLASH_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
pma_status pma_flash_attention_static(const pma_attn_params *p, const pma_layout *layout,
                                      const pma_bf16 *qh, const pma_bf16 *kh,
                                      const pma_bf16 *vt, pma_bf16 *o, int64_t o_ld, float *lse,
                                      void *stream);

/* Workspace of pma_attention: qh, kh and vt (3 * H * Lp * D bf16), then the
 * flash workspace (pma_flash_workspace_size). */
pma_status pma_attention_workspace_size(const pma_attn_params *p, int32_t seq_len,
                                        size_t *bytes);

/* pma_qk_norm_rope followed by pma_flash_attention; q, k, v are not modified. */
pma_status pma_attention(const pma_attn_params *p, const pma_layout *layout,
                         const pma_bf16 *q, int64_t q_ld, const pma_bf16 *k, int64_t k_ld,
                         const pma_bf16 *v, int64_t v_ld, const float *q_norm_weight,
                         const float *k_norm_weight, pma_bf16 *o, int64_t o_ld, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream);


/* ======================================================================
 * 3. DiT block: AdaLN table, LN + modulate, projections, SwiGLU FFN
 * ----------------------------------------------------------------------
 * [H3] intro: one block stack over the packed sequence; modality-specific
 * behaviour comes only from the per-row modality tag selecting the AdaLN
 * modulation; the block stack is stored in bf16.  [H3] constructor
 * parameters: hidden_size (5376), ffn_dim (14336) of the SwiGLU feed-forward,
 * time_embed_dim (2688) = the input of every AdaLN projection, norm_eps
 * (1e-5) of the pre-attention and pre-feed-forward norms.  [ENG] "Exacte DiT
 * fusions": the gated residual is written as exact bf16 and the same row is
 * normalised for the next sublayer; "Profiling en diagnostische pads":
 * fc1 -> SwiGLU -> fc2.
 *
 * Readings of the pages' open points:
 *   table[g][t][k][c] = sum_e temb[t][e] * W_ada[g][k*hidden + c][e] (per
 *     tag g in {0 video, 1 text, 2 audio}; no bias, no activation), chunks
 *     k = 0..5: shift_a, scale_a, gate_a, shift_f, scale_f, gate_f;
 *   padding rows (tag -1) use all-zero modulation;
 *   a  = LN(x)  * (1 + scale_a) + shift_a      LN: no affine, population var
 *   [Q|K|V] = a W_qkv^T                         (attention path of section 2)
 *   x1 = x  + gate_a * (O W_o^T)
 *   b  = LN(x1) * (1 + scale_f) + shift_f
 *   h  = silu(b W_gate^T) * (b W_up^T)          W_fc1 rows = [gate | up]
 *   x2 = x1 + gate_f * (h W_fc2^T)
 * Weights are stored [out][in] (row j = the input weights of output j).
 * ====================================================================== */

typedef struct {
    int32_t hidden;          /* residual width; multiple of 256              */
    int32_t ffn_dim;         /* SwiGLU inner width; multiple of 128          */
    int32_t time_embed_dim;  /* E; multiple of 8                              */
    float norm_eps;          /* pre-norm epsilon                              */
    pma_attn_params attn;    /* num_heads * 128 must be a multiple of 256     */
} pma_block_params;

typedef struct {
    const pma_bf16 *w_ada;          /* [3][6*hidden][E]                     */
    const pma_bf16 *w_qkv;          /* [3*H*D][hidden]  Q heads | K | V      */
    const pma_bf16 *w_o;            /* [hidden][H*D]                         */
    const pma_bf16 *w_fc1;          /* [2*ffn][hidden]  gate rows | up rows  */
    const pma_bf16 *w_fc2;          /* [hidden][ffn]                         */
    const float *q_norm_weight;     /* [128]                                 */
    const float *k_norm_weight;     /* [128]                                 */
} pma_block_weights;

/* AdaLN modulation table.  temb: bf16 [T][E]; w_ada: bf16 [3][6*hidden][E];
 * table: fp32 [3][T][6][hidden].  T <= 8 and T * E <= 24576. */
pma_status pma_adaln_table(const pma_block_params *p, int32_t num_timesteps,
                           const pma_bf16 *temb, const pma_bf16 *w_ada, float *table,
                           void *stream);

/* out = LN(x) * (1 + scale) + shift per row, (shift, scale) gathered from
 * table by the row's (tag, timestep index); which = 0 selects chunks
 * (shift_a, scale_a), 1 selects (shift_f, scale_f).  x, out: bf16 [L][hidden]
 * (may alias). */
pma_status pma_ln_modulate(const pma_block_params *p, const pma_layout *layout,
                           const float *table, int32_t which, const pma_bf16 *x,
                           pma_bf16 *out, void *stream);

/* Epilogues of pma_linear. */
#define PMA_EPI_STORE         0 /* C = acc                                          */
#define PMA_EPI_GATE_RESIDUAL 1 /* C = R + gate * acc, gate = table chunk per row    */
#define PMA_EPI_SWIGLU        2 /* C[:, j] = silu(acc_gate[j]) * acc_up[j]           */

typedef struct {
    int32_t M;             /* rows of A and C                                        */
    int32_t N;             /* output columns (SWIGLU: columns of C = gate rows of W) */
    int32_t K;             /* reduction length; multiple of 64                       */
    const pma_bf16 *A; int64_t lda;    /* [M][K]                                    */
    const pma_bf16 *W; int64_t ldw;    /* [N][K]; SWIGLU: [2N][K], up rows at N..2N */
    pma_bf16 *C; int64_t ldc;          /* [M][N]                                    */
    int32_t epilogue;      /* PMA_EPI_*                                              */
    /* GATE_RESIDUAL only: */
    const pma_bf16 *R; int64_t ldr;    /* residual [M][N] (may alias C)             */
    const float *table;    /* [3][T][6][N] modulation table                          */
    int32_t num_timesteps; /* T                                                       */
    int32_t gate_chunk;    /* 2 (gate_a) or 5 (gate_f)                               */
    const int32_t *token_tags, *timestep_indices;   /* [M] per-row gather keys      */
} pma_linear_args;

/* C = epilogue(A W^T) in bf16 with fp32 accumulation on bf16 MFMA.
 * N % 256 == 0 (SWIGLU: N % 128 == 0), K % 64 == 0, lda/ldw/ldc/ldr % 8 == 0,
 * pointers 16-byte aligned, M * lda and the rows of W addressable in 32-bit
 * byte offsets (< 4 GiB).  Rows >= M are neither read nor written. */
pma_status pma_linear(const pma_linear_args *args, void *stream);

/* Device workspace of pma_gate_residual_ln_modulate for seq_len rows (the
 * rows' LayerNorm statistics: at most hidden / 128 fp32 pairs per row). */
pma_status pma_gate_ln_workspace_size(const pma_block_params *p, int32_t seq_len,
                                      size_t *bytes);

/* A gated residual fused with the next AdaLN norm.  [ENG] "Exacte DiT
 * fusions": the attention residual gate is fused with the following MLP
 * AdaLN, and the rounded row stays on chip for its norm.  Here:
 *   x1 = x + gate * (a w^T), rounded to bf16 once (pma_linear with the
 *        GATE_RESIDUAL epilogue, gate = gate_table chunk gate_chunk, 2 =
 *        gate_a or 5 = gate_f), whose epilogue also takes, from the rounded
 *        values in its registers, each row's mean and sum of squared
 *        deviations over the columns one wave holds (two passes);
 *   b  = LN(x1) * (1 + scale) + shift as pma_ln_modulate with mod_table and
 *        which, its mean and variance combined from those per-group pairs
 *        (Chan's pairwise update) instead of a reduction over the row.
 * x1 is bit-identical to pma_linear's GATE_RESIDUAL output; b equals
 * pma_ln_modulate(x1) up to the fp32 summation order of the statistics.
 * a: bf16 [L][K] (leading dimension lda), w: bf16 [hidden][K], x, x1, b:
 * bf16 [L][hidden] (x1 may alias x, b may alias x1); K % 64 == 0.  The two
 * tables may differ (the block's a7 -> a8 uses one table with gate_chunk 2
 * and which 1; a block's fc2 and the next block's first norm, gate_chunk 5
 * and which 0 with the next block's table).  workspace: at least
 * pma_gate_ln_workspace_size bytes, 256-byte aligned; it holds the
 * statistics between the two launches, so calls that share it must not
 * overlap. */
pma_status pma_gate_residual_ln_modulate(const pma_block_params *p, const pma_layout *layout,
                                         const pma_bf16 *a, int64_t lda, int32_t K,
                                         const pma_bf16 *w, const float *gate_table,
                                         int32_t gate_chunk, const pma_bf16 *x, pma_bf16 *x1,
                                         const float *mod_table, int32_t which, pma_bf16 *b,
                                         void *workspace, size_t workspace_bytes, void *stream);

/* (cos, sin) of every row's rotation angles for the fused QKV projection:
 * table fp32 [L][3F][2], entry [i][a*F + f] = (cos, sin) of
 * pos[i][a] * theta^(-f/F) (the angle of the attention section's RoPE),
 * computed in fp64 and rounded to fp32.  table 8-byte aligned. */
pma_status pma_rope_table(const pma_attn_params *p, const pma_layout *layout, float *table,
                          void *stream);

/* The QKV projection fused with QK-RMSNorm + 3-axis RoPE: from a (bf16
 * [L][hidden], leading dimension lda) and w_qkv ([3*H*D][hidden], Q rows,
 * then K, then V) it writes the operands pma_qk_norm_rope would write --
 * qh, kh [H][Lp][D] normalised and rotated, vt [H][D][Lp] -- without storing
 * Q, K, V: the norm and rotation read the fp32 accumulators (Q and K are
 * rounded to bf16 once, after rotation; qh carries the logit factor
 * softmax_scale * log2(e) as in pma_qk_norm_rope).  Rows L..Lp-1 are written
 * as zero.
 * H must be even (a 256-column tile never straddles Q, K and V); hidden %
 * 64 == 0; a, w_qkv, qh, kh, vt, the norm weights and rope_table (from
 * pma_rope_table) 16-byte aligned.
 * [ENG] "Checkpoint layout en media pipeline": the engine runs the QK
 * normalisation and RoPE as one fused kernel on the projection output. */
pma_status pma_qkv_projection(const pma_attn_params *p, const pma_layout *layout,
                              const pma_bf16 *a, int64_t lda, int32_t hidden,
                              const pma_bf16 *w_qkv, const float *q_norm_weight,
                              const float *k_norm_weight, const float *rope_table,
                              pma_bf16 *qh, pma_bf16 *kh, pma_bf16 *vt, void *stream);

/* Device workspace of pma_block_forward for L rows. */
pma_status pma_block_workspace_size(const pma_block_params *p, int32_t seq_len, size_t *bytes);

/* One DiT block: x_out = block(x_in).  table from pma_adaln_table; layout
 * built with the attention tiles.  x_in, x_out: bf16 [L][hidden], distinct.
 * The QKV projection is pma_qkv_projection (Q and K are never stored), so
 * the head count is even. */
pma_status pma_block_forward(const pma_block_params *p, const pma_layout *layout,
                             const pma_block_weights *w, const float *table,
                             const pma_bf16 *x_in, pma_bf16 *x_out, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Block stack.  [H3] constructor parameters: num_layers (50) blocks, each
 * with its own weights; [ENG] "Scheduling en activatiegeheugen": one
 * activation arena serves every block.  Reading: block l gets its own AdaLN
 * table temb W_ada[l]^T (computed just before it, into the workspace) and the
 * bf16 residual stream passes from block to block; the RoPE table is built
 * once per call.  w: host array of num_blocks weight sets (device pointers);
 * temb: bf16 [T][E] with T = layout->num_timesteps; x_in, x_out: bf16
 * [L][hidden], distinct.  Workspace: pma_stack_workspace_size, 256-byte
 * aligned, reused by every block. */
pma_status pma_stack_workspace_size(const pma_block_params *p, int32_t seq_len,
                                    int32_t num_timesteps, size_t *bytes);
pma_status pma_stack_forward(const pma_block_params *p, const pma_layout *layout,
                             int32_t num_blocks, const pma_block_weights *w,
                             const pma_bf16 *temb, const pma_bf16 *x_in, pma_bf16 *x_out,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Token refiner.  [H3] constructor parameters: num_refiner_layers (2)
 * blocks applied to the projected text stream, text_dim (5120) the width of
 * the text conditioning, final_norm_eps (1e-5) the epsilon of the refiner's
 * output norm.  Readings: proj = text W_text^T (bf16, no bias, as every
 * projection of the bf16 stack); then num_blocks blocks (pma_stack_forward)
 * over the text rows alone, described by text_layout (seq_len = n text rows,
 * every tag 1, the rows' own positions and timestep indices; built with
 * pma_layout_build and the attention tiles); then LayerNorm without affine,
 * eps = final_norm_eps.  text: bf16 [n][text_ld]; w_text: bf16
 * [hidden][text_dim], text_dim % 64 == 0; out: bf16 [n][hidden] (the rows
 * pma_pack_rows scatters to the text indices).  num_blocks may be 0. */
pma_status pma_refiner_workspace_size(const pma_block_params *p, int32_t n_text,
                                      int32_t num_timesteps, size_t *bytes);
pma_status pma_text_refiner(const pma_block_params *p, const pma_layout *text_layout,
                            int32_t num_blocks, const pma_block_weights *w,
                            const pma_bf16 *temb, const pma_bf16 *text, int64_t text_ld,
                            int32_t text_dim, const pma_bf16 *w_text, float final_norm_eps,
                            pma_bf16 *out, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Token reduction.  [ENG] presets and implementation notes: an optional
 * mode pairs adjacent horizontal target-video tokens after block 3, keeps
 * text, audio and reference tokens exact, and restores the full-resolution
 * state, kept as a bypass, before a later block (block 40 for the first ten
 * noisy evaluations, block 30 afterwards).  The caller builds the plan (as it
 * builds every layout): reduced row i stands for full rows src0[i] and
 * src1[i] (src1[i] = -1: src0[i] alone), every full row named exactly once;
 * and the reduced layout, whose merged rows sit at w + 1/2 (positions in
 * half units with pos_scale 1/2 on every axis).  Readings:
 *   merge:   xr[i] = src1[i] < 0 ? x[src0[i]] : bf16((x[src0[i]] + x[src1[i]]) / 2)
 *   restore: x_out[r] = bf16(bypass[r] + (xr_after[i] - xr_before[i])) for
 *            r in {src0[i], src1[i]}: the change the reduced blocks made to
 *            merged row i goes to both of its rows.
 * Rows are bf16 [.][hidden], hidden % 8 == 0, 16-byte aligned; x_out may
 * alias bypass.  The kernels trust the plan's contents as far as memory
 * safety goes: an entry outside [0, seq_len) is skipped (merge writes that
 * reduced row as zeros), and a full row named twice is restored twice.
 * pma_token_plan_check verifies a plan on the device once, before use. */
pma_status pma_token_merge(int32_t hidden, int32_t seq_len, int32_t n_reduced,
                           const int32_t *src0, const int32_t *src1, const pma_bf16 *x,
                           pma_bf16 *xr, void *stream);
pma_status pma_token_restore(int32_t hidden, int32_t seq_len, int32_t n_reduced,
                             const int32_t *src0, const int32_t *src1, const pma_bf16 *bypass,
                             const pma_bf16 *xr_before, const pma_bf16 *xr_after,
                             pma_bf16 *x_out, void *stream);

/* Check a token-reduction plan on the device: every src0 entry and every src1
 * entry other than -1 inside [0, seq_len), and every full row named by
 * exactly one entry.  workspace: device int32 [seq_len + 3], overwritten.
 * Synchronises the stream and copies the verdict back: *bits (host) gets the
 * PMA_PLAN_* bits, *first_bad_entry the first reduced row with a bad index
 * (-1: none), *first_bad_row the first full row named by no entry or by
 * several (-1: none).  Returns PMA_ERR_LAYOUT when any bit is set. */
#define PMA_PLAN_BAD_INDEX     (1 << 0) /* src0 outside [0, L), or src1 outside and not -1 */
#define PMA_PLAN_ROW_MISSING   (1 << 1) /* a full row that no entry names                 */
#define PMA_PLAN_ROW_REPEATED  (1 << 2) /* a full row named by more than one entry        */
pma_status pma_token_plan_check(int32_t seq_len, int32_t n_reduced, const int32_t *src0,
                                const int32_t *src1, int32_t *workspace, void *stream,
                                int32_t *bits, int32_t *first_bad_entry, int32_t *first_bad_row);

/* ======================================================================
 * 4. Input and output path: timestep MLP, row pack, output heads
 * ----------------------------------------------------------------------
 * [H3] constructor parameters: freq_dim (256) of the sinusoidal timestep
 * embedding, timesteps taken unscaled in [0, 1]; time_embed_hidden_dim
 * (5376) and time_embed_dim (2688), the timestep MLP's inner and output
 * widths; in_channels * prod(patch_size) (24 * 4 = 96) and audio_in_channels
 * (32), the widths of the latent rows; final_norm_eps (1e-5) of norm_out.
 * [H3] forward parameters: the video, audio and text rows arrive ordered as
 * video_indices, audio_indices and text_indices; timestep holds the distinct
 * values and timestep_indices points each row into it.  [H3] returns: the
 * video and audio velocities in the row order of their index tensors.  [H3]
 * intro: the patch projections, the timestep MLP and the two output heads
 * are fp32.  [ENG] "Exacte DiT fusions": the fp32 patch projections round
 * straight to bf16 into the packed hidden stream; the final audio/video
 * AdaLN reads its rows at their offsets in the residual stream and the
 * heads modulate while loading their projection tiles.
 *
 * Readings of the pages' open points:
 *   e(t) = [cos(t w_j) | sin(t w_j)], w_j = max_period^(-j / half),
 *     half = freq_dim / 2, j = 0..half-1, max_period 10000;
 *   temb = W2 silu(W1 e + b1) + b2                (fp32)
 *   x[idx[i]] = bf16(rows[i] W^T + b)             video and audio rows
 *   x[text_idx[i]] = text[i]                      projected text rows (bf16)
 *   head m (0 video, 1 audio): (shift, scale) = temb[ts] W_mod[m]^T, no bias,
 *     out[i] = (LN(x[idx[i]]) * (1 + scale) + shift) W_out^T + b_out (fp32),
 *     LN without affine, population variance, eps = final_norm_eps, ts the
 *     row's timestep index.
 * Weights are fp32 [out][in].
 * ====================================================================== */

typedef struct {
    int32_t freq_dim;      /* sinusoid width: multiple of 4, 4..2048        */
    int32_t inner_dim;     /* time_embed_hidden_dim: multiple of 4          */
    int32_t embed_dim;     /* time_embed_dim E: multiple of 4                 */
    float max_period;      /* > 1 (10000)                                     */
} pma_temb_params;

/* Timestep MLP for T <= 8 distinct timesteps.  timestep: fp32 [T];
 * w1 [inner][freq_dim], b1 [inner], w2 [E][inner], b2 [E] fp32;
 * inner: fp32 [T][inner] (written; the MLP's hidden activation);
 * temb: fp32 [T][E]; temb_bf16 (optional, may be NULL): the same values
 * rounded to bf16, the input pma_adaln_table takes.  Weights and activations
 * 16-byte aligned. */
pma_status pma_timestep_embed(const pma_temb_params *p, int32_t num_timesteps,
                              const float *timestep, const float *w1, const float *b1,
                              const float *w2, const float *b2, float *inner, float *temb,
                              pma_bf16 *temb_bf16, void *stream);

typedef struct {
    int32_t hidden;          /* packed stream width: multiple of 128, <= 8192   */
    int32_t video_channels;  /* video row width: multiple of 32 (96)            */
    int32_t audio_channels;  /* audio row width: multiple of 32 (32)            */
    int32_t video_out;       /* video head width: multiple of 32, <= 128 (96)   */
    int32_t audio_out;       /* audio head width: multiple of 32, <= 128 (32)   */
    int32_t time_embed_dim;  /* E: multiple of 4                                */
    float final_norm_eps;    /* >= 0 (1e-5)                                     */
} pma_io_params;

/* Write the input rows into the packed stream x (bf16 [seq_len][hidden]):
 * video_rows fp32 [num_video][video_channels] through w_video
 * [hidden][video_channels] + b_video, audio_rows likewise, and the projected
 * text rows (bf16, row stride text_ld >= hidden) copied.  desc supplies
 * seq_len and the device index arrays (counts may be 0, pointers then
 * ignored).  Rows named by no index are not written; index entries outside
 * [0, seq_len) are skipped (pma_layout_build flags them).  Indices must be
 * distinct.  fp32 arrays and x 16-byte aligned; text_ld % 8 == 0. */
pma_status pma_pack_rows(const pma_io_params *p, const pma_layout_desc *desc,
                         const float *video_rows, const float *w_video, const float *b_video,
                         const float *audio_rows, const float *w_audio, const float *b_audio,
                         const pma_bf16 *text_rows, int64_t text_ld, pma_bf16 *x,
                         void *stream);

/* Output-head modulation table: table[m][t][k][c] = sum_e temb[t][e] *
 * w_mod[m][k*hidden + c][e], k = 0 shift, 1 scale.  temb fp32 [T][E];
 * w_mod fp32 [2][2*hidden][E]; table fp32 [2][T][2][hidden].  T <= 8. */
pma_status pma_head_table(const pma_io_params *p, int32_t num_timesteps, const float *temb,
                          const float *w_mod, float *table, void *stream);

/* Device workspace of pma_unpack_rows for the given row counts. */
pma_status pma_unpack_workspace_size(const pma_io_params *p, int32_t num_video,
                                     int32_t num_audio, size_t *bytes);

/* Output heads: video_out fp32 [num_video][video_out] and audio_out fp32
 * [num_audio][audio_out] from the rows of x (bf16 [seq_len][hidden]) named by
 * desc's video and audio indices, in index order.  table from
 * pma_head_table with T = desc->num_timesteps (<= 8); w_video_out
 * [video_out][hidden], w_audio_out [audio_out][hidden] and the biases fp32.
 * A row whose timestep index is outside [0, T) is not modulated; an index
 * entry outside [0, seq_len) yields a row equal to the bias.  All arrays
 * 16-byte aligned; workspace >= pma_unpack_workspace_size, 256-byte aligned. */
pma_status pma_unpack_rows(const pma_io_params *p, const pma_layout_desc *desc,
                           const pma_bf16 *x, const float *table, const float *w_video_out,
                           const float *b_video_out, const float *w_audio_out,
                           const float *b_audio_out, float *video_out, float *audio_out,
                           void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PMA_H_ */
