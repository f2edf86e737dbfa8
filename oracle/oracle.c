/*
 * CPU oracle for the packed masked attention path of the MiniMax-H3 DiT block.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is plain, slow, obviously correct C.
 * Only tests/, the smoke check in __graft_entry__.py and the cpu_baseline leg
 * of bench.py load it.  It shares no code, header, table or constant with the
 * HIP library under packed_masked_attention_amd/csrc, and the HIP library
 * never calls it.
 *
 * Sources (pages cited by title and section):
 *  [H3]  "MiniMaxH3Transformer3DModel" (diffusers API page):
 *        intro (packed 1-D sequence, full self-attention, padding rows with
 *        tag -1 kept in their own attention document by a boolean mask),
 *        constructor parameters (attention_head_dim, rope_freq_dim,
 *        rope_theta, qk_norm_eps), class description (original reference pads
 *        and splits the tail into its own varlen document),
 *        forward parameters (token_tags, position_ids, timestep_indices,
 *        video/audio/text index tensors).
 *
 * Readings of points the pages leave open (each listed in the design doc):
 *  - per-head query/key norm = RMSNorm over the head's channels, eps inside
 *    the root, one weight vector of head_dim entries shared by all heads;
 *  - norm first, then RoPE;
 *  - inv_freq[f] = theta^(-f/F), f = 0..F-1, shared by the t, h, w axes;
 *  - axis a in {t,h,w} rotates channels [2aF, 2aF+2F) in rotate-half pairs
 *    (2aF+f, 2aF+f+F) by angle pos[a]*inv_freq[f], direction e^{+i phi};
 *    channels >= 6F pass through unchanged;
 *  - softmax scale 1/sqrt(head_dim), no bias, no causal mask;
 *  - pair (i, j) may attend iff [tag_i == -1] == [tag_j == -1]: every padding
 *    row sits in one padding document, every other row in the other one.
 *
 * Nothing here parallelises beyond independent (row, head) items; there is no
 * blocking, no online softmax and no reordering of the definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* bf16 storage format                                                 */
/* ------------------------------------------------------------------ */

/* bf16 bit pattern -> exact double (bf16 is the top half of an IEEE single). */
double oracle_bf16_value(uint16_t bits)
{
    union { uint32_t u; float f; } x;
    x.u = ((uint32_t)bits) << 16;
    return (double)x.f;
}

void oracle_bf16_to_f64(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_value(in[i]);
}

/*
 * Round a double to the nearest bf16 value, ties to even, computed directly
 * from the definition: bf16 keeps 8 significant bits and the fp32 exponent
 * range (normal exponents -126..127, subnormal step 2^-133).
 */
uint16_t oracle_bf16_round(double v)
{
    union { uint32_t u; float f; } x;
    if (isnan(v)) return 0x7fc0;
    double a = fabs(v);
    if (a == 0.0) { x.f = (float)v; return (uint16_t)(x.u >> 16); }
    int e;
    frexp(a, &e);                 /* a = m * 2^e, 0.5 <= m < 1 */
    int ulp_exp = e - 8;          /* 8 significant bits */
    if (ulp_exp < -133) ulp_exp = -133;
    double q = ldexp(a, -ulp_exp);            /* exact: power-of-two scale */
    double r = nearbyint(q);                  /* default mode: ties to even */
    double rv = ldexp(r, ulp_exp);
    if (rv > 3.3895313892515355e38) rv = INFINITY;   /* above bf16 max -> inf */
    x.f = (float)(v < 0 ? -rv : rv);          /* exact in fp32 */
    return (uint16_t)(x.u >> 16);
}

void oracle_bf16_round_array(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(in[i]);
}

/* ------------------------------------------------------------------ */
/* Layout: validation, documents, tile classes ([H3] intro, forward)   */
/* ------------------------------------------------------------------ */

/* Status bits of a packed layout.  The same bit meanings are documented in
 * the library header; each side implements them from that definition. */
#define OR_BAD_TAG        (1 << 0)  /* tag not in {-1, 0, 1, 2}                  */
#define OR_BAD_TIMESTEP   (1 << 1)  /* non-padding row with index outside [0,T)  */
#define OR_BAD_POSITION   (1 << 2)  /* |position| >= 2^24                         */
#define OR_BAD_INDEX      (1 << 3)  /* index tensor entry outside [0, L)          */
#define OR_UNSORTED_INDEX (1 << 4)  /* index tensor not strictly ascending        */
#define OR_INDEX_TAG      (1 << 5)  /* index points at a row of another modality  */
#define OR_INDEX_COUNT    (1 << 6)  /* index count != number of rows of that tag  */

static int check_index(const int32_t *idx, int32_t n, int32_t L,
                       const int32_t *tags, int32_t want_tag, int32_t *tag_count)
{
    int st = 0;
    for (int32_t i = 0; i < n; ++i) {
        int32_t r = idx[i];
        if (r < 0 || r >= L) { st |= OR_BAD_INDEX; continue; }
        if (i > 0 && !(idx[i - 1] < r)) st |= OR_UNSORTED_INDEX;
        if (tags[r] != want_tag) st |= OR_INDEX_TAG;
    }
    int32_t cnt = 0;
    for (int32_t r = 0; r < L; ++r) cnt += (tags[r] == want_tag);
    if (cnt != n) st |= OR_INDEX_COUNT;
    *tag_count = cnt;
    return st;
}

/*
 * Validate the packed layout of [H3] forward parameters.  Tags: 0 video,
 * 1 text, 2 audio ([H3] forward, token_tags), -1 padding ([H3] intro).
 * Returns the OR of the status bits; *err_row gets the smallest row with a
 * per-row error (bad tag, timestep index or position), or -1.
 */
int32_t oracle_layout_status(int32_t L, int32_t T, const int32_t *tags,
                             const int32_t *pos, const int32_t *ts_idx,
                             const int32_t *video_idx, int32_t nv,
                             const int32_t *audio_idx, int32_t na,
                             const int32_t *text_idx, int32_t nt,
                             int32_t *err_row)
{
    int32_t st = 0, first = -1;
    for (int32_t i = 0; i < L; ++i) {
        int32_t row_bits = 0;
        int32_t t = tags[i];
        if (!(t == -1 || t == 0 || t == 1 || t == 2)) row_bits |= OR_BAD_TAG;
        if (t != -1 && (ts_idx[i] < 0 || ts_idx[i] >= T)) row_bits |= OR_BAD_TIMESTEP;
        for (int a = 0; a < 3; ++a) {
            int64_t p = pos[3 * (int64_t)i + a];
            if (p <= -(1 << 24) || p >= (1 << 24)) row_bits |= OR_BAD_POSITION;
        }
        if (row_bits && first < 0) first = i;
        st |= row_bits;
    }
    int32_t c;
    st |= check_index(video_idx, nv, L, tags, 0, &c);
    st |= check_index(audio_idx, na, L, tags, 2, &c);
    st |= check_index(text_idx, nt, L, tags, 1, &c);
    *err_row = first;
    return st;
}

/* Document id of every row: 1 for padding (tag -1), 0 otherwise. */
void oracle_layout_doc(int32_t L, const int32_t *tags, int32_t *doc)
{
    for (int32_t i = 0; i < L; ++i) doc[i] = (tags[i] == -1) ? 1 : 0;
}

/* May row i attend to row j?  Same document. */
static int allowed(const int32_t *tags, int32_t i, int32_t j)
{
    return (tags[i] == -1) == (tags[j] == -1);
}

/*
 * Tile classes of the (BM x BN) tiling of the L x L attention mask, by brute
 * force over every in-range pair of every tile: 0 EMPTY (no allowed pair),
 * 2 FULL (every pair allowed), 1 PARTIAL otherwise.  cls is [nqt][nkt].
 * count[qt] = number of non-EMPTY k-tiles of q-tile qt; list[qt][0..count)
 * are those k-tiles in ascending order (rest of the row left -1).
 * order[] lists q-tiles by descending count, ties by ascending index.
 */
void oracle_layout_tiles(int32_t L, const int32_t *tags, int32_t BM, int32_t BN,
                         uint8_t *cls, int32_t *count, int32_t *list,
                         int32_t *order)
{
    int32_t nqt = (L + BM - 1) / BM, nkt = (L + BN - 1) / BN;
#pragma omp parallel for schedule(dynamic)
    for (int32_t qt = 0; qt < nqt; ++qt) {
        int32_t n = 0;
        for (int32_t kt = 0; kt < nkt; ++kt) {
            int64_t pairs = 0, ok = 0;
            for (int32_t i = qt * BM; i < (qt + 1) * BM && i < L; ++i)
                for (int32_t j = kt * BN; j < (kt + 1) * BN && j < L; ++j) {
                    ++pairs;
                    ok += allowed(tags, i, j);
                }
            uint8_t c = (ok == 0) ? 0 : (ok == pairs ? 2 : 1);
            cls[(int64_t)qt * nkt + kt] = c;
            list[(int64_t)qt * nkt + kt] = -1;
            if (c != 0) list[(int64_t)qt * nkt + n++] = kt;
        }
        count[qt] = n;
    }
    /* rank of each q-tile in (count desc, index asc) order */
    for (int32_t a = 0; a < nqt; ++a) {
        int32_t rank = 0;
        for (int32_t b = 0; b < nqt; ++b)
            if (count[b] > count[a] || (count[b] == count[a] && b < a)) ++rank;
        order[rank] = a;
    }
}

/* Number of allowed (i, j) pairs: sum over documents of n_d^2. */
int64_t oracle_allowed_pairs(int32_t L, const int32_t *tags)
{
    int64_t npad = 0;
    for (int32_t i = 0; i < L; ++i) npad += (tags[i] == -1);
    return npad * npad + (L - npad) * (L - npad);
}

/* ------------------------------------------------------------------ */
/* QK-RMSNorm + 3-axis RoPE ([H3] constructor parameters)              */
/* ------------------------------------------------------------------ */

/* inv_freq[f] = theta^(-f/F): the frequency buffer shared by t, h and w. */
void oracle_inv_freq(int32_t F, double theta, double *inv_freq)
{
    for (int32_t f = 0; f < F; ++f) inv_freq[f] = pow(theta, -(double)f / (double)F);
}

/*
 * x: [L][ld] values with head h of row i at x[i*ld + h*D + c].
 * y: fp64 [L][H][D].  For every (row, head):
 *   r = 1/sqrt(mean_c x_c^2 + eps);  n_c = x_c * r * w[c]
 *   for axis a, f < F: phi = (pos[i][a] * pos_scale[a]) * inv_freq[f];
 *     c0 = 2aF+f; c1 = c0+F
 *     y_c0 = n_c0 cos phi - n_c1 sin phi;  y_c1 = n_c1 cos phi + n_c0 sin phi
 *   y_c = n_c for c >= 6F.
 * pos_scale (3 values; NULL = all 1) scales each axis' coordinate: the
 * engine page's 256x256 preview halves the spatial (h, w) coordinates, which
 * makes the effective positions fractional.
 */
void oracle_qk_norm_rope(int32_t L, int32_t H, int32_t D, int32_t F, double theta,
                         double eps, const double *x, int64_t ld, const double *w,
                         const int32_t *pos, const double *pos_scale, double *y)
{
    double inv_freq[64];
    oracle_inv_freq(F, theta, inv_freq);
#pragma omp parallel for schedule(static)
    for (int64_t item = 0; item < (int64_t)L * H; ++item) {
        int64_t i = item / H, h = item % H;
        const double *xr = x + i * ld + h * D;
        double *yr = y + (i * H + h) * D;
        double ss = 0.0;
        for (int32_t c = 0; c < D; ++c) {
            ss += xr[c] * xr[c];
        }
        double r = 1.0 / sqrt(ss / D + eps);
        double n[1024];
        for (int32_t c = 0; c < D; ++c) n[c] = xr[c] * r * w[c];
        for (int32_t c = 0; c < D; ++c) yr[c] = n[c];
        for (int32_t a = 0; a < 3; ++a) {
            double p = (double)pos[3 * i + a] * (pos_scale ? pos_scale[a] : 1.0);
            for (int32_t f = 0; f < F; ++f) {
                double phi = p * inv_freq[f];
                int32_t c0 = 2 * a * F + f, c1 = c0 + F;
                yr[c0] = n[c0] * cos(phi) - n[c1] * sin(phi);
                yr[c1] = n[c1] * cos(phi) + n[c0] * sin(phi);
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Masked softmax attention ([H3] intro, class description)            */
/* ------------------------------------------------------------------ */

/*
 * Two-pass exact softmax attention for the listed query rows, every head.
 * q, k, v: [L][H][D] (REAL); o: [nrows][H][D]; lse: [nrows][H] (nullable).
 *   s_j = scale * <q_i, k_j> if doc(i) == doc(j) else -inf
 *   p_j = exp(s_j - max s) / sum exp(s - max s);  o_i = sum_j p_j v_j
 *   lse_i = max s + log(sum exp(s - max s))
 * Instantiated for double (parity) and float (CPU timing baseline).
 */
#define DEFINE_ATTENTION(NAME, REAL, EXP, LOG)                                       \
void NAME(int32_t L, int32_t H, int32_t D, const REAL *q, const REAL *k,             \
          const REAL *v, const int32_t *tags, double scale, const int32_t *rows,     \
          int32_t nrows, REAL *o, REAL *lse)                                         \
{                                                                                    \
    _Pragma("omp parallel")                                                          \
    {                                                                                \
        REAL *s = (REAL *)malloc(sizeof(REAL) * (size_t)L);                          \
        _Pragma("omp for schedule(dynamic)")                                         \
        for (int64_t item = 0; item < (int64_t)nrows * H; ++item) {                  \
            int64_t r = item / H, h = item % H;                                      \
            int32_t i = rows[r];                                                     \
            const REAL *qi = q + ((int64_t)i * H + h) * D;                           \
            REAL mx = -INFINITY;                                                     \
            for (int32_t j = 0; j < L; ++j) {                                        \
                if (!allowed(tags, i, j)) { s[j] = -INFINITY; continue; }            \
                const REAL *kj = k + ((int64_t)j * H + h) * D;                       \
                REAL acc = 0;                                                        \
                for (int32_t c = 0; c < D; ++c) acc += qi[c] * kj[c];                \
                s[j] = acc * (REAL)scale;                                            \
                if (s[j] > mx) mx = s[j];                                            \
            }                                                                        \
            REAL sum = 0;                                                            \
            for (int32_t j = 0; j < L; ++j) {                                        \
                s[j] = (s[j] == -INFINITY) ? 0 : EXP(s[j] - mx);                     \
                sum += s[j];                                                         \
            }                                                                        \
            REAL *oi = o + (r * H + h) * D;                                          \
            for (int32_t c = 0; c < D; ++c) oi[c] = 0;                               \
            for (int32_t j = 0; j < L; ++j) {                                        \
                if (s[j] == 0) continue;                                             \
                const REAL *vj = v + ((int64_t)j * H + h) * D;                       \
                REAL pj = s[j] / sum;                                                \
                for (int32_t c = 0; c < D; ++c) oi[c] += pj * vj[c];                 \
            }                                                                        \
            if (lse) lse[r * H + h] = mx + LOG(sum);                                 \
        }                                                                            \
        free(s);                                                                     \
    }                                                                                \
}

DEFINE_ATTENTION(oracle_attention_f64, double, exp, log)
DEFINE_ATTENTION(oracle_attention_f32, float, expf, logf)

/* Number of OpenMP threads the oracle runs on. */
int32_t oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
