/*
 * ridgefill.h -- C ABI of the RidgeFill ridge fit and late-layer KV-cache fill for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes (RidgeFill project page, "Method" steps 1-4 and Figure 2(b); "Abstract"):
 * the lower layers of a model run exactly up to a split layer; for every filled prompt row
 * and every late layer, a per-layer ridge map fitted once in closed form predicts that
 * layer's input from the split layer's state, and the layer's own K/V projections write its
 * cache from the prediction.  The same fit serves the KV-Lingo page's token-wise cache
 * translators (section 3.2, closed-form first stage), whose maps rf_translate applies.  The order of the layer's own cache path follows the KV-Lingo
 * page, section 3.1 "Rotation and normalisation" (pre-norm storing: normalise, project,
 * rotate keys by position, store).
 *
 * Conventions for every entry point
 *  - Pointers named d_* are device memory of the current HIP device, owned by the caller.
 *    Arrays of pointers (``const void* const*``) are host arrays of device pointers.
 *    The library allocates no device memory and keeps no state between calls.
 *  - ``stream`` is a hipStream_t (NULL = the null stream).  Every call only enqueues work on
 *    it and returns without synchronising.
 *  - Arguments are validated on the host before anything is enqueued.  On a failed check the
 *    call returns RF_ERR_INVALID_ARG or RF_ERR_UNSUPPORTED, enqueues nothing, and
 *    rf_last_error() (thread-local) describes the problem.
 *  - RF_ERR_HIP means a launch failed; rf_last_error() holds the HIP error string.
 *  - Row-vector notation: a token state is x in R^{1 x d}.  Matrices are row-major.
 *  - Weight matrices are stored out-feature major ("Linear" layout): a map W stored as
 *    [d_out][d_in] computes y = x W^T.  This puts the reduction dimension contiguous for
 *    both operands of every GEMM.
 *  - bf16 is IEEE bfloat16 stored as 16-bit words; conversions round to nearest even.
 *  - Calls on one stream are ordered; calls that write the same buffers from different
 *    streams race.
 */
#ifndef RIDGEFILL_H
#define RIDGEFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RF_OK = 0,
    RF_ERR_INVALID_ARG = 1,   /* a null pointer, bad size, bad range or bad stride        */
    RF_ERR_UNSUPPORTED = 2,   /* a valid request the library does not implement (shape)  */
    RF_ERR_HIP = 3,           /* a HIP runtime call or kernel launch failed               */
    RF_ERR_WORKSPACE = 4,     /* the workspace passed is smaller than the size query says */
    RF_ERR_NOT_SPD = 5        /* a regularised Gram is not positive definite (reported by
                                 rf_info_status from the pivots rf_solve left on the device) */
} rf_status;

typedef enum { RF_F32 = 0, RF_BF16 = 1 } rf_dtype;
typedef enum { RF_LAYOUT_CONTIGUOUS = 0, RF_LAYOUT_PAGED = 1 } rf_layout;
typedef enum {
    RF_LAMBDA_ABSOLUTE = 0,      /* lambda added to the centred Gram's diagonal as given       */
    RF_LAMBDA_REL_MEAN_DIAG = 1  /* lambda x mean diagonal of the centred Gram (KV-Lingo,
                                    Appendix B.2 "Protocol", relative ridge convention)      */
} rf_lambda_mode;

/* Library version string, e.g. "ridgefill 0.1.0 gfx950". */
const char* rf_version(void);

/* Text of the last error raised on the calling thread ("" if none). */
const char* rf_last_error(void);

/* ---------------------------------------------------------------------------------------
 * Ridge fit, part 1: one streaming pass of second moments over calibration chunks.
 *
 * RidgeFill project page, "Method" step 2 and "Abstract": the map of each late layer is a
 * ridge regression fitted once, in closed form, from one pass over calibration rows.  The
 * pass carries, for the split-layer rows X ([rows][d]) and each target's rows Y_l
 * ([rows][m], m = d_out, or d when d_out is 0):
 *     n        number of rows seen                       (int64)
 *     S_xx   = X^T X                 [d][d]               (fp32; rows <= cols are defined,
 *                                                          the strict lower triangle is not)
 *     S_yx   = Y_l^T X for each l    [n_targets*m][d]     (fp32; row l*m+o, column i holds
 *                                                          sum_r Y_l[r][o] X[r][i])
 *     s_x    = 1^T X                 [d]                  (fp64)
 *     s_y    = 1^T Y_l for each l    [n_targets*m]        (fp64)
 *     s_yy   = 1^T (Y_l * Y_l)       [n_targets*m]        (fp64 column sums of squares: the
 *                                                          fit's R^2 is read off the state)
 * The state is one device buffer laid out as rf_gram_state_layout() reports; it is plain
 * data, so it can be copied out and back to checkpoint and resume a calibration pass.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    int32_t d;          /* width of the X rows (the maps' input); a multiple of 256  */
    int32_t n_targets;  /* number of target layers whose inputs are regressed on X  */
    rf_dtype dtype;     /* dtype of the X and Y rows passed to rf_gram_accumulate   */
    int32_t d_out;      /* width m of each target's Y rows (the maps' output); 0 = d,
                           else a multiple of 256, at most 65536                    */
} rf_gram_desc;

typedef struct {       /* byte offsets into the state buffer */
    int64_t off_n, off_S_xx, off_S_yx, off_s_x, off_s_y, off_s_yy, total_bytes;
} rf_gram_layout_t;

/* Host only.  Fills *out; returns RF_ERR_INVALID_ARG for a bad descriptor. */
rf_status rf_gram_state_layout(const rf_gram_desc* desc, rf_gram_layout_t* out);

/* Host only.  Bytes of the state buffer (0 for a bad descriptor). */
size_t rf_gram_state_bytes(const rf_gram_desc* desc);

/* Zero the state (n = 0, all sums 0).  d_state: rf_gram_state_bytes() bytes, 256-B aligned. */
rf_status rf_gram_init(const rf_gram_desc* desc, void* d_state, void* stream);

/* Add one chunk of ``rows`` calibration rows to the state.
 *  d_X : [rows][ldx] split-layer rows, dtype desc->dtype, ldx >= d, 16-B aligned rows
 *  d_Y : host array of n_targets device pointers, each [rows][ldy] target-layer input rows,
 *        ldy >= m
 *  rows: >= 0 (0 is a no-op).  Any row count is allowed; ragged tails are handled.  The rows
 *        are read in place (no workspace); a chunk whose byte offsets would pass 2^31 is
 *        taken in several pieces.
 * Results are deterministic: the same chunks in the same order give bit-identical sums. */
rf_status rf_gram_accumulate(const rf_gram_desc* desc, void* d_state,
                             const void* d_X, int64_t ldx,
                             const void* const* d_Y, int64_t ldy,
                             int64_t rows, void* stream);

/* Sub-state of column blocks of X, for fits from a subset of source layers (KV-Lingo page,
 * section 3.1, greedy match: forward selection over source layers, each candidate set fitted
 * from the one accumulated pass).  X's d columns form d / block_width blocks (block_width a
 * multiple of 256 that divides d); blocks (host, n_sel in 1..64, strictly ascending) selects
 * some.  d_state_out (laid out for desc_out: d = n_sel * block_width, the same n_targets,
 * d_out and dtype; distinct from d_state) receives n, S_xx over the selected blocks (their
 * upper triangle; the rest of the tile rows is copied as it lies), the selected columns of
 * S_yx and s_x, and s_y, s_yy unchanged: exactly the state one pass over the selected
 * columns alone would have left.  Solving it gives the maps from the selected blocks alone. */
rf_status rf_gram_select(const rf_gram_desc* desc, const void* d_state, int32_t block_width,
                         const int32_t* blocks, int32_t n_sel, const rf_gram_desc* desc_out,
                         void* d_state_out, void* stream);

/* ---------------------------------------------------------------------------------------
 * Ridge fit, part 2: the closed-form solve, for one Gram and a batch of ridge strengths.
 *
 * For each lambda_z of the batch and each selected target l (intercept by mean-centring, rows
 * as token states):
 *     mu_x = s_x / n,  mu_l = s_y,l / n
 *     C    = S_xx - n mu_x^T mu_x           (centred Gram, symmetric from the upper triangle)
 *     B_l  = S_yx,l - n mu_l^T mu_x          (centred cross moments, [m][d])
 *     W_l  = B_l (C + lambda_z I)^-1         (out-feature major: row o is the map of output o)
 *     b_l  = mu_l - mu_x W_l^T
 * so that the prediction is y = x W_l^T + b_l.  Every C + lambda_z I = L L^T is factored by
 * Cholesky in fp64, the factorisations of the batch advancing together (one launch per
 * diagonal block for all of them), and inverted in fp64 (L^-T by recursive doubling over
 * diagonal blocks, then the lower triangle of L^-T L^-1, mirrored where read).
 *
 * The product B_l (C + lambda_z I)^-1 has two routes:
 *  - split bf16: on the bf16 matrix cores in three-term split precision (each factor,
 *    equilibrated by D = diag(C + lambda_0 I), is split into two bf16 parts) with fp32
 *    accumulation: about 1e-5 of max |W_l| from the fp64 product while the equilibrated
 *    inverse D^1/2 (C + lambda I)^-1 D^1/2 has entries of order one, and worse in proportion
 *    to its largest entry (near-collinear features with lambda far below their variance);
 *  - fp64: the product in fp64 on the matrix cores (about 30x the time of the split route).
 * RF_PRODUCT_AUTO takes the split route and, for each lambda whose equilibrated inverse has an
 * entry above RF_SPLIT_COND_MAX, writes the maps again from the fp64 route; the choice is made
 * on the device (no synchronisation), and d_cond reports the largest entry.
 *
 *  lambdas : host array of n_lambda (1..8) ridge strengths, each >= 0 and finite
 *  targets : host array of n_sel target indices in [0, n_targets)
 *  product : RF_PRODUCT_AUTO, RF_PRODUCT_SPLIT_BF16 or RF_PRODUCT_F64
 *  d_W     : [n_lambda][n_sel][m][d] fp32 out, may be NULL; 16-B aligned
 *  d_W_lp  : [n_lambda][n_sel][m][d] bf16 out, may be NULL; 16-B aligned.  Written in the
 *            fill's packed layout (as rf_pack_weights with rope_head_dim 0 would leave it),
 *            ready for rf_fill
 *  d_b     : [n_lambda][n_sel][m] fp32 out, may be NULL
 *  d_info  : [n_lambda] int32 out: 0 = success; k > 0 = C + lambda_z I is not positive
 *            definite and the k-th leading minor (1-based) is the first that fails.  That
 *            lambda's outputs are then meaningless (finite or not) but every write stays in
 *            bounds.  rf_info_status() turns a host copy into RF_OK / RF_ERR_NOT_SPD.
 *  d_cond  : [n_lambda] fp64 out, may be NULL: the largest |entry| of the equilibrated inverse
 *            (1 for uncorrelated features; +inf when it holds a NaN)
 *  d_resid : [n_lambda][n_sel] fp64 out, may be NULL: the stationarity residual of the maps
 *            written, max |(C + lambda I) W_l^T - B_l^T| / max |B_l|, from d_W in fp64 against
 *            C and B_l rebuilt from the state (needs d_W; costs one fp64 product of the
 *            product's size per lambda)
 *  d_ws    : rf_solve_workspace_bytes(desc, n_sel, n_lambda) bytes, 256-B aligned
 * ------------------------------------------------------------------------------------- */
typedef enum {
    RF_PRODUCT_AUTO = 0,        /* split bf16; fp64 for a lambda whose d_cond > RF_SPLIT_COND_MAX */
    RF_PRODUCT_SPLIT_BF16 = 1,  /* split bf16 always                                             */
    RF_PRODUCT_F64 = 2          /* fp64 always                                                   */
} rf_product;
#define RF_SPLIT_COND_MAX 8.0
#define RF_MAX_LAMBDAS 8

size_t rf_solve_workspace_bytes(const rf_gram_desc* desc, int32_t n_sel, int32_t n_lambda);
rf_status rf_solve(const rf_gram_desc* desc, const void* d_state,
                   const double* lambdas, int32_t n_lambda, rf_lambda_mode mode,
                   const int32_t* targets, int32_t n_sel, rf_product product,
                   float* d_W, void* d_W_lp, float* d_b,
                   int32_t* d_info, double* d_cond, double* d_resid,
                   void* d_ws, size_t ws_bytes, void* stream);

/* Head-wise maps.  KV-Lingo page, section 3.1 "Head mixing" (a head-wise translator maps each
 * source head only onto the same target head: its map is block-diagonal by head) and section
 * 3.2 (the first stage fits the maps in closed form).  The ridge fit restricted to such maps is
 * one independent ridge fit per head: target head h on head h of every source layer.  Computed
 * as rf_solve with the centred moments between different heads taken as zero, so that the
 * regularised system is block-diagonal by head and its solution is those per-head maps; the
 * blocks between heads of the output are exactly zero.  Features are numbered as the state
 * has them: target output o belongs to head o / head_dim; source feature i, of source layer
 * i / d_out, to head (i % d_out) / head_dim (source layers of the targets' layout side by side).
 *  head_dim : a positive multiple of 8 dividing the targets' width d_out; d a multiple of d_out
 * Every other argument, output and workspace as for rf_solve (rf_solve_workspace_bytes). */
rf_status rf_solve_headwise(const rf_gram_desc* desc, const void* d_state,
                            const double* lambdas, int32_t n_lambda, rf_lambda_mode mode, int32_t head_dim,
                            const int32_t* targets, int32_t n_sel, rf_product product,
                            float* d_W, void* d_W_lp, float* d_b,
                            int32_t* d_info, double* d_cond, double* d_resid,
                            void* d_ws, size_t ws_bytes, void* stream);

/* Host only.  RF_OK when all n pivots reports (a host copy of rf_solve's d_info) are 0, else
 * RF_ERR_NOT_SPD with the first failing lambda and pivot in rf_last_error(). */
rf_status rf_info_status(const int32_t* info, int32_t n);

/* The same maps by the symmetric eigendecomposition route (KV-Lingo page, appendix on the
 * training procedure, "Stage 1": the per-layer normal equations solved once by symmetric
 * eigendecomposition, eigenvalues below a relative tolerance counting as zero).  C + lambda I = V diag(mu) V^T by cyclic Jacobi in fp64
 * (``sweeps`` sweeps of round-robin rotations; 15 reach fp64 accuracy on the widths used here);
 * A^+ keeps 1/mu_i for mu_i > rel_tol * max mu; then W_l = B_l A^+ and b_l as in rf_solve (its
 * split-bf16 route).  For a regular system this is rf_solve's map; for a singular one
 * (lambda = 0 on rank-deficient rows: low-rank caches, duplicated or constant features) it is
 * the minimum-norm least-squares map, where rf_solve reports a failed pivot.  Outputs and
 * their layouts as for rf_solve (no d_info: the route has no pivot to fail).
 *  d_ws : rf_solve_pinv_workspace_bytes(desc, n_sel) bytes, 256-B aligned
 * Needs rel_tol in [0, 1), sweeps in [1, 64]; one kernel pair per Jacobi round (d - 1 rounds
 * per sweep), so it suits offline fits of widths up to a few thousand. */
size_t rf_solve_pinv_workspace_bytes(const rf_gram_desc* desc, int32_t n_sel);
rf_status rf_solve_pinv(const rf_gram_desc* desc, const void* d_state, double lambda,
                        rf_lambda_mode mode, double rel_tol, int32_t sweeps,
                        const int32_t* targets, int32_t n_sel,
                        float* d_W, void* d_W_lp, float* d_b, void* d_ws, size_t ws_bytes,
                        void* stream);

/* ---------------------------------------------------------------------------------------
 * Fit quality.  KV-Lingo page, Appendix "The R^2 assignment": the score of a map is the
 * fraction of its target's features it explains, read off the sums the fit accumulated (no
 * extra pass over the data).  For each selected target l, with W_l the fp32 map rf_solve
 * returned for the same state, lambda and mode:
 *     B_l   = S_yx,l - s_y,l s_x^T / n                 (centred cross moments, [m][d])
 *     SST_l = sum_o (s_yy,l[o] - s_y,l[o]^2 / n)        (centred total sum of squares)
 *     R^2_l = (sum_{o,i} W_l[o][i] B_l[o][i] + lambda' sum_{o,i} W_l[o][i]^2) / SST_l
 * where lambda' is the absolute ridge strength (lambda, or lambda x the mean diagonal of the
 * centred Gram).  For the exact ridge map this equals 1 - ||Y~ - X~ W_l^T||^2 / ||Y~||^2 on
 * the centred rows.  Sums run in fp64 in a fixed order.
 *  targets : host array of n_sel target indices in [0, n_targets)
 *  d_W     : [n_sel][m][d] fp32, 16-B aligned
 *  d_r2    : [n_sel] fp64 out
 *  d_ws    : rf_fit_r2_workspace_bytes(desc, n_sel) bytes, 256-B aligned
 * ------------------------------------------------------------------------------------- */
size_t rf_fit_r2_workspace_bytes(const rf_gram_desc* desc, int32_t n_sel);
rf_status rf_fit_r2(const rf_gram_desc* desc, const void* d_state, double lambda, rf_lambda_mode mode,
                    const int32_t* targets, int32_t n_sel, const float* d_W, double* d_r2,
                    void* d_ws, size_t ws_bytes, void* stream);

/* Host only.  The R^2 assignment (KV-Lingo page, Appendix "The R^2 assignment"): for each
 * target layer l, the nu source layers s with the highest r2[l * n_src + s] (host fp64
 * [n_tgt][n_src], e.g. rf_fit_r2 of single-source fits), written to out[l * nu + j] (host
 * int32 [n_tgt][nu]) in ascending layer order.  Equal scores go to the shallower layer; NaN
 * scores rank last.
 * Keys and values are ranked apart by calling it once per side.  Needs 1 <= nu <= n_src. */
rf_status rf_r2_assignment(const double* r2, int32_t n_tgt, int32_t n_src, int32_t nu, int32_t* out);

/* ---------------------------------------------------------------------------------------
 * KV cache layout (host only).
 *
 * Each filled layer has one K pool and one V pool of the same shape.
 *  CONTIGUOUS: [max_tokens][n_kv_heads][head_dim]; token t lives in row t.
 *  PAGED     : [n_blocks][n_kv_heads][block_size][head_dim] with
 *              n_blocks = ceil(max_tokens / block_size); token t lives in physical block
 *              block_table[t / block_size], slot t % block_size (serving systems keep KV in
 *              pages: RIFT page, section 4.1, "Block-Level RIFT-stat").
 * Strides are in elements.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t block_size;   /* PAGED only; ignored for CONTIGUOUS */
    int64_t max_tokens;   /* tokens the pool holds */
    rf_layout layout;
    rf_dtype dtype;       /* element type of the pool */
} rf_cache_desc;

typedef struct {
    int64_t n_blocks;         /* PAGED: physical blocks; CONTIGUOUS: max_tokens */
    int64_t elem_bytes;
    int64_t bytes_per_pool;   /* bytes of one K (or one V) pool of one layer */
    int64_t stride_block;     /* PAGED only (0 for CONTIGUOUS) */
    int64_t stride_head;
    int64_t stride_token;
} rf_cache_layout_t;

rf_status rf_cache_layout(const rf_cache_desc* desc, rf_cache_layout_t* out);

/* ---------------------------------------------------------------------------------------
 * RoPE table.  KV-Lingo page, section 2: RoPE rotates keys by their token's position.
 * Rotate-half convention: within each head the pair (i, i + head_dim/2) turns by
 * pos * base^(-2i/head_dim).  Writes d_table[pos][i] = (cos, sin) as two fp32 for
 * pos in [0, n_pos), i in [0, head_dim/2).  Angles and their cos/sin are evaluated in fp64
 * and rounded once to fp32, so the table stays accurate at positions beyond 10^5.
 * ------------------------------------------------------------------------------------- */
rf_status rf_rope_table(double base, int32_t head_dim, int64_t n_pos, float* d_table,
                        void* stream);
/* Workspace bytes a fill given no RoPE table uses for the table of n_tokens positions. */
size_t rf_rope_workspace_bytes(int32_t head_dim, int64_t n_tokens);

/* ---------------------------------------------------------------------------------------
 * Weight packing for the fill's matrix-core products (a layout change, no arithmetic).
 * The bf16 fill reads its weight rows (map, K and V projections) straight into the
 * matrix-core operand registers, so they are stored in fragment order; grouping the K/V rows
 * by rotate-half pairs puts both members of a RoPE pair (KV-Lingo page, section 2) in one
 * thread.  Copies a row-major [rows][ld_src] matrix of element type ``dtype`` (BF16 copied
 * as is, F32 rounded to nearest even bf16) into the bf16 buffer d_dst
 * (rows * cols elements, no padding) as consecutive 256-row tiles; within a tile, element
 * (r, k) (r the row in the tile) moves to
 *     (k/64)*16384 + (r'/64)*4096 + ((k%64)/16)*1024 + ((r'%64)/32)*512
 *     + (((k%16)/8)*32 + r'%32)*8 + k%8
 * where r' is the packed position of row r: r' = r when rope_head_dim is 0.  Otherwise the
 * rows of each tile are grouped by rotate-half pairs: packed row r' = 64w + 32i + j
 * (w, i, j in [0,4), [0,2), [0,32)) holds tile row (q / h) * hd + q % h + i * h with
 * q = 32w + j, hd = rope_head_dim, h = hd / 2 (pair partners i = 0, 1 share w and j).
 * Supported: BF16 or F32 sources, rows % 256 == 0, cols % 64 == 0, rows and cols <= 65536,
 * rope_head_dim in {0, 64, 128}; ld_src >= cols and a multiple of 8; both buffers 16-B
 * aligned and disjoint.
 * Asynchronous on ``stream``; nothing is allocated.
 * ------------------------------------------------------------------------------------- */
rf_status rf_pack_weights(rf_dtype dtype, int64_t rows, int64_t cols, const void* d_src, int64_t ld_src,
                          int32_t rope_head_dim, void* d_dst, void* stream);

/* ---------------------------------------------------------------------------------------
 * Weight-only int8 maps.  RidgeFill project page, "Code, data and maps" (the ridge maps on
 * Hugging Face): some published maps are int8; the page gives no scheme, and this is the
 * reading taken: symmetric codes per output row.  For each row o of the fp32 map d_W
 * ([rows][ld], row-major, out-feature major as rf_solve writes it), in fp32:
 *     s_o = max_i |W[o][i]| / 127,   q[o][i] = round_half_even(W[o][i] / s_o) in [-127, 127]
 * (a row of zeros: s_o = 0, q_o = 0).  The codes go to d_q (rows * cols bytes) in the packed
 * order of rf_pack_weights with rope_head_dim 0, one byte per element; the scales to
 * d_scale ([rows] fp32).  Half the bytes of a bf16 map for the fill's map product (which then
 * applies diag(s) q): the streamed fill copies half as much.  Maps must be finite.
 * Supported: rows % 256 == 0, cols % 64 == 0, rows and cols <= 65536, ld >= cols and a multiple
 * of 4, d_W and d_scale 16-B aligned, d_q 16-B aligned.  Asynchronous on ``stream``; nothing
 * is allocated.
 * ------------------------------------------------------------------------------------- */
rf_status rf_quantize_map(int64_t rows, int64_t cols, const float* d_W, int64_t ld, void* d_q, float* d_scale,
                          void* stream);

/* ---------------------------------------------------------------------------------------
 * The fill.  RidgeFill project page, "Method" steps 2-4 and Figure 2(b): for every token
 * t in [t0, t1) and every listed late layer l,
 *     h = x_t W_l^T + b_l                              (predicted layer input)
 *     u = h / sqrt(mean_j h_j^2 + rms_eps) * gamma_l   (the layer's own RMSNorm)
 *     k = u W_k,l^T,  v = u W_v,l^T                    (the layer's own K/V projections)
 *     k <- k_g / sqrt(mean(k_g^2) + k_norm_eps) * k_norm_l  for each head g  (only when
 *          k_norm is given: models that normalise keys per head, KV-Lingo page, section 2)
 *     k <- RoPE(k, pos0 + t)                           (keys only)
 * and k, v are stored in the layer's K and V pools at token t.  Rows outside [t0, t1) and
 * layers not listed are never written: exact rows skip the map (project page, Fig. 2).
 *
 * Weights, per listed layer (host arrays of n_layers device pointers):
 *   W_map[l] : [d][d]                dtype    out-feature major map; BF16 maps in the packed
 *                                             layout of rf_pack_weights (rope_head_dim 0)
 *   b_map[l] : [d]                   fp32
 *   gamma[l] : [d]                   fp32
 *   W_k[l]   : [n_kv_heads*head_dim][d] dtype  head-major output rows; BF16 packed by
 *   W_v[l]   : [n_kv_heads*head_dim][d] dtype  rf_pack_weights with rope_head_dim = head_dim
 * d_X : rows of the split-layer state for tokens t0..t1-1 (row i is token t0+i), [t1-t0][ldx]
 * k_cache[l], v_cache[l] : pools laid out per *cache (dtype must equal weights->dtype)
 * d_block_table : PAGED only, int32 [n_table_blocks]; entries outside [0, n_blocks) are
 *                 skipped (their tokens are not written)
 * d_rope : rf_rope_table() output with rope_len >= pos0 + t1 positions, head_dim of *cache;
 *          or NULL: the table of positions pos0 + t0 .. pos0 + t1 - 1 is then built from
 *          weights->rope_base (the same fp64 angles as rf_rope_table) at the end of d_ws, which
 *          must hold rf_rope_workspace_bytes(head_dim, t1 - t0) bytes more (likewise for
 *          rf_fill_composed, rf_fill_static and rf_fill_streamed; rope_len is then unused)
 * d_ws   : rf_fill_workspace_bytes(weights, t1 - t0) bytes, 256-B aligned
 * Supported: d % 256 == 0, head_dim in {64, 128}, (n_kv_heads*head_dim) % 256 == 0,
 * dtype F32 or BF16 (all of X, maps, projections and pools share it).
 * Weight-only int8 maps (map_scale non-NULL, BF16 only): W_map[l] holds int8 codes in the
 * packed order of rf_quantize_map (one byte per element) and map_scale[l] ([d] fp32, 16-B
 * aligned) their row scales; the fill applies the map diag(map_scale[l]) codes, i.e.
 *     h = (x codes^T) * map_scale + b_map        (the codes widened to bf16 exactly)
 * and everything after h is as above.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    int32_t d;
    int32_t n_kv_heads;
    int32_t head_dim;
    float rms_eps;
    rf_dtype dtype;
    const void* const* W_map;
    const float* const* b_map;
    const float* const* gamma;
    const void* const* W_k;
    const void* const* W_v;
    const float* const* k_norm;   /* NULL, or per layer fp32 [head_dim]: per-head key norm    */
    float k_norm_eps;             /* its epsilon (inside the root), when k_norm is given      */
    const float* const* map_scale; /* NULL, or per layer fp32 [d]: W_map are int8 codes       */
    double rope_base;             /* RoPE base: used only when a fill is given no rope table   */
} rf_fill_weights;

size_t rf_fill_workspace_bytes(const rf_fill_weights* weights, int64_t max_rows);
rf_status rf_fill(const rf_fill_weights* weights, int32_t n_layers,
                  const void* d_X, int64_t ldx,
                  int64_t t0, int64_t t1, int64_t pos0,
                  const rf_cache_desc* cache, void* const* k_cache, void* const* v_cache,
                  const int32_t* d_block_table, int64_t n_table_blocks,
                  const float* d_rope, int64_t rope_len,
                  void* d_ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * The composed fill: the same caches as rf_fill, from the maps folded into the layers' own
 * projections once per map.  RidgeFill project page, "Method" steps 2-4: only the K/V rows
 * of a filled layer are written, and the predicted input h = x W^T + b enters them only
 * through its RMS and its projections, so for a map W, b and a layer's gamma, W_k, W_v
 *     k = (x M_k^T + c_k) r,   v = (x M_v^T + c_v) r,   r = 1/sqrt(mean_o h_o^2 + rms_eps)
 * with M_k = W_k diag(gamma) W, c_k = W_k diag(gamma) b (likewise for v), and
 *     sum_o h_o^2 = sum_i x_i ((T x^T)_i + g_i x_i) + x q_lin^T + q_const,
 *     T = the strict upper triangle of 2 W^T W, g = the diagonal of W^T W (kept in fp32),
 *     q_lin = 2 W^T b, q_const = |b|^2,
 * then the per-head key norm (if given) and RoPE on k as in rf_fill.  Per token and layer the
 * products take 2 d (d/2 + 2 H_kv d_h) + O(d) FLOP instead of rf_fill's 2 d (d + 2 H_kv d_h):
 * the map's own product becomes a triangular quadratic form, and the projections read the
 * prompt states directly.
 *
 * rf_fill_compose forms the composed weights of n_layers layers from rf_fill's (BF16, packed)
 * weights.  Per layer l (device buffers, caller-owned, 16-B aligned):
 *   T[l]   : [d][d] bf16 out, packed as a map (rope_head_dim 0); only the blocks on and above
 *            the 256 x 256 block diagonal are written or read
 *   q[l]   : [2d + 1] fp32 out: q_lin, then g, then q_const
 *   M_k[l], M_v[l] : [n_kv_heads*head_dim][d] bf16 out, packed as rf_pack_weights with
 *            rope_head_dim = head_dim packs W_k, W_v
 *   c_k[l], c_v[l] : [n_kv_heads*head_dim] fp32 out
 * Products of bf16 weights accumulate in fp32 (W_k diag(gamma) enters in two bf16 parts, so
 * its product with W is exact to fp32 before the one rounding of M to bf16); the vectors are
 * summed in fp64.  d_ws: a multiple k >= 1 of rf_fill_compose_workspace_bytes(weights) bytes
 * (one layer slot: 2 d^2 + 8 H_kv d_h d bytes), 256-B aligned; the products of up to
 * min(k, 32) layers share one launch.
 * Supported: BF16 weights, d % 256 == 0, as for rf_fill.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    int32_t d;
    int32_t n_kv_heads;
    int32_t head_dim;
    float rms_eps;
    const void* const* T;
    const float* const* q;
    const void* const* M_k;
    const void* const* M_v;
    const float* const* c_k;
    const float* const* c_v;
    const float* const* k_norm;   /* NULL, or per layer fp32 [head_dim] (as for rf_fill)        */
    float k_norm_eps;
    double rope_base;             /* RoPE base: used only when a fill is given no rope table   */
} rf_fill_composed_weights;

size_t rf_fill_compose_workspace_bytes(const rf_fill_weights* weights);
rf_status rf_fill_compose(const rf_fill_weights* weights, int32_t n_layers,
                          void* const* T, float* const* q, void* const* M_k, void* const* M_v,
                          float* const* c_k, float* const* c_v,
                          void* d_ws, size_t ws_bytes, void* stream);

/* The fill from composed weights; arguments as for rf_fill (X, cache, block table, RoPE table,
 * rows outside [t0, t1) and layers not listed never written).  BF16 only.
 * d_ws: rf_fill_composed_workspace_bytes(weights, t1 - t0) bytes, 256-B aligned (per-token
 * partial sums of squares: d/256 fp32 per token and layer slot; more slots, more layers per
 * launch, up to 32). */
size_t rf_fill_composed_workspace_bytes(const rf_fill_composed_weights* weights, int64_t max_rows);
rf_status rf_fill_composed(const rf_fill_composed_weights* weights, int32_t n_layers,
                           const void* d_X, int64_t ldx,
                           int64_t t0, int64_t t1, int64_t pos0,
                           const rf_cache_desc* cache, void* const* k_cache, void* const* v_cache,
                           const int32_t* d_block_table, int64_t n_table_blocks,
                           const float* d_rope, int64_t rope_len,
                           void* d_ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * rf_fill without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Computes exactly what rf_fill computes (the same kernels, bit-identical caches) with its
 * workspace in a static device buffer of RF_FILL_STATIC_SCRATCH_MB MiB that the library holds
 * on every GPU it runs on until the process ends; the call itself allocates nothing.  A call
 * whose one-layer workspace (rf_fill_workspace_bytes(weights, t1 - t0), plus
 * rf_rope_workspace_bytes(head_dim, t1 - t0) without a rope table) exceeds the buffer is
 * refused with RF_ERR_UNSUPPORTED and nothing enqueued: fill such a range in several calls.
 * The buffer is shared by every call on one GPU and keeps the last call's contents (nothing
 * in it needs to start at zero); calls that overlap on one GPU (different streams, different
 * threads without ordering) race on it.  Other arguments as for rf_fill.
 * ------------------------------------------------------------------------------------- */
#define RF_FILL_STATIC_SCRATCH_MB 96
size_t rf_fill_static_scratch_bytes(void);
rf_status rf_fill_static(const rf_fill_weights* weights, int32_t n_layers,
                         const void* d_X, int64_t ldx,
                         int64_t t0, int64_t t1, int64_t pos0,
                         const rf_cache_desc* cache, void* const* k_cache, void* const* v_cache,
                         const int32_t* d_block_table, int64_t n_table_blocks,
                         const float* d_rope, int64_t rope_len, void* stream);

/* ---------------------------------------------------------------------------------------
 * Streamed maps.  RidgeFill project page, Figure 10 and Table 8 ("streamed"): the ridge maps
 * stay in host memory and reach the GPU layer by layer while the fill runs, for far less
 * device memory than resident maps at nearly the same speed.  Computes exactly what rf_fill
 * computes (the same kernels, bit-identical results), with W_map[l] HOST pointers to the
 * maps in the layout rf_fill takes (BF16 packed, or int8 codes with device map_scale), in
 * page-locked memory (hipHostMalloc) so the copies run asynchronously.  Every other weight is a device pointer as for rf_fill.
 *  d_ring      : device buffer of ring_bytes >= rf_fill_streamed_ring_bytes() bytes, 256-B
 *                aligned: ring_slots slots of layers_per_slot maps
 *  d_ws        : rf_fill_workspace_bytes(weights, rows) * layers_per_slot bytes, rows = the
 *                tokens filled per step: rows_per_fill, or t1 - t0 when it is 0 (or larger)
 *  rows_per_fill : 0, or the tokens of [t0, t1) filled per step: a long prompt is filled in
 *                steps of this many tokens inside each layer chunk, so each map is copied once
 *                per call however many steps the range takes (the workspace covers one step)
 *  copy_stream : a stream other than ``stream`` (hipStream_t) for the host-to-device copies
 * Layers go in chunks of layers_per_slot (1..32): chunk c is copied into slot
 * c % ring_slots on copy_stream once the fill of chunk c - ring_slots has left that slot, and
 * filled on ``stream`` once its copy has landed (HIP events order the two streams; they are
 * created and released inside the call).  The call's first copy waits for everything enqueued
 * on ``stream`` before the call, so consecutive calls on one stream (a long prompt filled in
 * token chunks) are ordered like any other calls on it.  Two or more slots let the copy of one
 * chunk run under the fill of the previous one.  The host maps must stay valid until ``stream``
 * reaches the end of the call's work.
 * ------------------------------------------------------------------------------------- */
size_t rf_fill_streamed_ring_bytes(const rf_fill_weights* weights, int32_t ring_slots, int32_t layers_per_slot);
rf_status rf_fill_streamed(const rf_fill_weights* weights, int32_t n_layers,
                           const void* d_X, int64_t ldx,
                           int64_t t0, int64_t t1, int64_t pos0,
                           const rf_cache_desc* cache, void* const* k_cache, void* const* v_cache,
                           const int32_t* d_block_table, int64_t n_table_blocks,
                           const float* d_rope, int64_t rope_len,
                           void* d_ws, size_t ws_bytes,
                           void* d_ring, size_t ring_bytes, int32_t ring_slots, int32_t layers_per_slot,
                           int64_t rows_per_fill, void* stream, void* copy_stream);

/* ---------------------------------------------------------------------------------------
 * Gated DeltaNet state update.  RidgeFill project page, "Method" step 3 and Figure 2(b): on a
 * Gated DeltaNet (linear-attention) layer the filled rows also run the layer's own state
 * update, from the keys, values and gates its projections make of the predicted input.  The
 * page does not write the update out; this is the published Gated DeltaNet recurrence (Yang,
 * Kautz and Hatamizadeh, "Gated Delta Networks", 2024), per layer and head:
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 * with S in R^{d_v x d_k} (fp32), over tokens t = 0 .. n_tokens-1 in order, starting from the
 * state in d_state and leaving the final state there: a prompt filled in chunks continues
 * from the previous chunk's state.  With normalise_k the keys are first scaled to unit length
 * per head, k / sqrt(|k|^2 + eps).  Arithmetic in fp32 (keys and values upcast exactly).
 * Per listed layer (host arrays of n_layers device pointers):
 *   d_k[l], d_v[l]   : [n_tokens][ld_k], [n_tokens][ld_v] rows, dtype; head h's key is
 *                      elements h d_k .. h d_k + d_k - 1 of its row (values likewise)
 *   d_g[l], d_beta[l]: [n_tokens][n_heads] fp32 log decay (<= 0) and write strength
 *   d_state[l]       : [n_heads][d_v][d_k] fp32, in and out, 16-B aligned
 * Supported: d_k in {64, 128}, d_v <= 4096, up to 64 layers per call.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    int32_t n_heads;
    int32_t d_k;
    int32_t d_v;
    rf_dtype dtype;        /* of the key and value rows                       */
    int32_t normalise_k;   /* 1: unit-length keys per head before the update  */
    float eps;             /* inside the root of the key norm                 */
} rf_gdn_desc;

rf_status rf_gdn_state(const rf_gdn_desc* desc, int32_t n_layers,
                       const void* const* d_k, const void* const* d_v, int64_t ld_k, int64_t ld_v,
                       const float* const* d_g, const float* const* d_beta, int64_t n_tokens,
                       float* const* d_state, void* stream);

/* ---------------------------------------------------------------------------------------
 * Token-wise linear KV-cache translators.  KV-Lingo page, section 3.1 "Linear translator
 * family": each target layer l has its own linear map for keys and its own for values, both
 * reading the cache rows of a set of nu source layers; with pre-norm storing the maps act on
 * the source keys before rotation, and the translated keys are rotated by their token's
 * position before they are stored.  For every token t in [t0, t1) and listed target layer l,
 *     k = s_k T_k,l^T + b_k,l,   v = s_v T_v,l^T + b_v,l
 *     k <- k_g / sqrt(mean(k_g^2) + k_norm_eps) * k_norm_l  for each head g  (when given)
 *     k <- RoPE(k, pos0 + t)                           (keys only)
 * and k, v are stored in the layer's K and V pools at token t.  s_k (s_v) is the row of
 * token t in d_src_k[l] (d_src_v[l]): the keys before rotation (the values) of the layer's
 * nu source layers side by side, d_in = nu * d_src wide.  A source cache kept as
 * [token][source layer][d_src] hands over a band of consecutive source layers (the bands of
 * rf_relative_depth_sources) as one row segment, with ld_src = n_src_layers * d_src.
 * Head-mixing maps are dense (headwise = 0).  A head-wise map (block-diagonal: target head g
 * reads only head g of each source layer, so the source heads match the target's and
 * d_in = nu * n_kv_heads * head_dim) is passed dense, zero blocks included; with headwise = 1
 * the BF16 product reads only the 256 x 256 blocks that hold a head's block (the entries
 * outside the head blocks must be zero: they are not all read), the F32 product reads all.  The maps'
 * closed-form first stage (KV-Lingo page, section 3.2) is a ridge fit of target rows on
 * source rows: rf_gram_accumulate and rf_solve with X = source rows, one target of the
 * same width; rf_pack_weights packs the solve's fp32 maps (rope_head_dim = head_dim).
 *
 * Maps, per listed target layer (host arrays of n_layers device pointers):
 *   T_k[l], T_v[l] : [n_kv_heads*head_dim][d_in] dtype, head-major output rows, out-feature
 *                    major; BF16 packed by rf_pack_weights with rope_head_dim = head_dim
 *   b_k, b_v       : both NULL (no intercept), or host arrays of n_layers fp32
 *                    [n_kv_heads*head_dim] device vectors, 16-B aligned
 * d_src_k[l], d_src_v[l] : [t1-t0][ld_src] source rows of tokens t0..t1-1 (row i is token
 *                    t0+i), dtype of the maps, 16-B aligned, ld_src a 16-byte multiple
 * cache, k_cache, v_cache, d_block_table, d_rope : as for rf_fill; rows outside [t0, t1)
 *                    and layers not listed are never written.  d_rope may be NULL: the keys
 *                    are then stored unrotated (post-RoPE translators, section 3.1, whose
 *                    maps act on keys the source already rotated; post-norm translators pass
 *                    the table and no k_norm)
 * No workspace.  Supported: d_in % 128 == 0 (BF16) or % 64 == 0 (F32), d_in <= 65536,
 * ld_src <= 2^21, head_dim in {64, 128}, (n_kv_heads*head_dim) % 256 == 0.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    int32_t d_in;
    int32_t n_kv_heads;
    int32_t head_dim;
    rf_dtype dtype;
    const void* const* T_k;
    const void* const* T_v;
    const float* const* b_k;
    const float* const* b_v;
    int32_t headwise;             /* 1: block-diagonal maps (see above); 0: dense maps          */
    const float* const* k_norm;   /* NULL, or per layer fp32 [head_dim]: the target's per-head
                                     key norm, applied after the map and before the rotation */
    float k_norm_eps;
} rf_translate_weights;

rf_status rf_translate(const rf_translate_weights* weights, int32_t n_layers,
                       const void* const* d_src_k, const void* const* d_src_v, int64_t ld_src,
                       int64_t t0, int64_t t1, int64_t pos0,
                       const rf_cache_desc* cache, void* const* k_cache, void* const* v_cache,
                       const int32_t* d_block_table, int64_t n_table_blocks,
                       const float* d_rope, int64_t rope_len, void* stream);

/* Host only.  Relative-depth match, KV-Lingo page, section 3.1 "Source-layer selection":
 * target layer l (1-based) reads the band of nu consecutive source layers centred on
 * c(l) = 1 + (l - 1)(n_src - 1)/(n_tgt - 1), shifted at the ends so every band holds nu
 * layers.  The band taken is the one whose middle is nearest c(l); an exact tie goes to the
 * deeper band; n_tgt = 1 reads c = 1.  Writes out[l * nu + j] (host int32 [n_tgt][nu]) = the
 * 0-based source layer j of 0-based target layer l.  Needs n_tgt >= 1, 1 <= nu <= n_src. */
rf_status rf_relative_depth_sources(int32_t n_src, int32_t n_tgt, int32_t nu, int32_t* out);

#ifdef __cplusplus
}
#endif

#endif /* RIDGEFILL_H */
