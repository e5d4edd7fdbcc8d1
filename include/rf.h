/*
 * rf.h - late-layer KV cache fill for AMD MI355X (gfx950).
 *
 * The operation is the cache fill of "RidgeFill: Training-Free Late-Layer
 * Cache Fill for Faster Prefill" (arXiv 2611.09709).  Layers below a split run
 * exactly.  For every prompt row outside the exact set (section 2.1: the tail
 * plus chosen prefix rows) and every late layer l, the fill
 *
 *   1. predicts the layer's input from the split state:  y = A_l x_S + b_l
 *      (section 2.2, the map equation);
 *   2. applies the layer's own RMSNorm:  h = gamma_l * y / sqrt(mean(y^2) + eps)
 *      (section 2.2: the prediction is normalised and projected exactly as a
 *      true input would be);
 *   3. applies its key and value projections:  k = W_k h,  v = W_v h
 *      (sections 2.1-2.2: for a filled row a late layer produces only the
 *      cache entries that later tokens attend to);
 *   4. rotates k with RoPE at the row's own position (section 2.2; section 6.6);
 *   5. stores bf16 k and v in that layer's cache slot for the row.  Exact rows
 *      are not touched (section 2.1; Figure 5, first sweep).
 *
 * Conventions for every call
 *  - bf16 values are passed as uint16_t bit patterns.  Matrices are row-major.
 *  - Pointers are device memory unless the comment says HOST.  The caller owns
 *    all memory; the library never frees a caller pointer.
 *  - Device work is enqueued on the caller's HIP stream (`hip_stream`, a
 *    hipStream_t; NULL = the default stream).  A call returns RF_OK once its
 *    work is enqueued; device faults surface at the caller's next sync.
 *  - Argument, shape and workspace errors are detected on the host before
 *    anything is enqueued; then nothing is written.  rf_last_error() returns a
 *    thread-local message for the last non-OK status.
 *  - rf_fill, rf_kv_project and rf_fill_rows allocate no device memory: all
 *    scratch comes from the caller's workspace.
 *  - With maps in device memory and no in-fill value measurement, rf_fill and
 *    rf_fill_q8 issue only kernel launches on hip_stream (no memory sets,
 *    events or synchronisation) and keep no state between calls, so they may
 *    be captured in a HIP graph and replayed.
 *  - Calls that share a plan must be issued from one host thread at a time.
 *
 * Layouts (per late layer l, all bf16):
 *    x       [n_rows][ld_x]               split state x_S, first d_in columns used
 *    map_a   [d_out][d_in]                A_l, row n = output feature n (the
 *                                         paper's orientation, section 2.2,
 *                                         y = A_l x + b_l).  For the row-vector
 *                                         form Y = X W_l + b_l, A_l = W_l^T: a
 *                                         caller holding W_l [d_in][d_out] passes
 *                                         its transpose.  rf_ridge_fit and
 *                                         rf_ridge_dev_solve return A_l.
 *    map_b   [d_out]                      b_l
 *    gamma   [d_out]                      RMSNorm gain
 *    w_k,w_v [n_kv*head_dim][d_out]       projection weights, [out][in]
 *    k_cache, v_cache [n_slots][n_kv][head_dim]
 *  RoPE: rotate-half.  Within each head, dimension j < head_dim/2 is paired
 *  with j + head_dim/2 and the pair is turned by pos * theta^(-2j/head_dim).
 */
#ifndef RF_H
#define RF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rf_status {
  RF_OK = 0,
  RF_E_ARG = -1,        /* null pointer, bad flag, bad count                     */
  RF_E_SHAPE = -2,      /* a dimension the kernels do not support               */
  RF_E_ROWS = -3,       /* RF_VALIDATE found bad fill rows, positions or slots   */
  RF_E_WORKSPACE = -4,  /* workspace too small or misaligned                     */
  RF_E_HIP = -5,        /* a HIP runtime call failed (message in rf_last_error)  */
  RF_E_LINALG = -6      /* ridge system not positive definite                    */
} rf_status;

/* rf_plan_create flags */
enum {
  RF_MAPS_HOST = 1, /* map_a/map_b given to rf_fill are pinned HOST pointers; they are
                       streamed to the GPU on a side stream, the first layer
                       alone and then up to RF_STREAM_GROUP layers per launch
                       group, each group's copy overlapped with the previous
                       group's fill (section 4.2: maps resident or streamed,
                       identical outputs)                                     */
  RF_VALIDATE = 2,  /* rf_fill / rf_kv_project check their row indices on the
                       device and synchronise the stream before launching     */
  RF_MAPS_Q8 = 4    /* maps are int8 with bf16 block scales and are passed to
                       rf_fill_q8 instead of rf_fill; d_in % 128 == 0 (see the
                       int8 map section below)                                 */
};

/* Most late layers one launch group takes when the maps are streamed
 * (RF_MAPS_HOST): the plan's two device map buffers hold this many layers
 * each.  Wider groups mean fewer, fuller launches; the first group is one
 * layer so that only one layer's copy precedes the first launch. */
#define RF_STREAM_GROUP 4

/* rf_ridge_solve / rf_ridge_fit flags */
enum {
  RF_RIDGE_RAW = 1 /* W = (X^T X + lambda I)^(-1) X^T Y, no centring, no offset */
};

typedef struct rf_shape {
  int32_t d_in;        /* width of the split state x_S; multiple of 64            */
  int32_t d_out;       /* width of a late layer's input; multiple of 256          */
  int32_t n_late;      /* late layers (layers from the split up); >= 1            */
  int32_t n_kv;        /* key/value heads per layer                              */
  int32_t head_dim;    /* 64 or 128; n_kv*head_dim must be a multiple of 128     */
  float rms_eps;       /* RMSNorm epsilon (inside the square root); >= 0         */
  double rope_theta;   /* RoPE base theta; > 1                                   */
  int32_t n_rows;      /* rows of x (all prompts of a batch concatenated)        */
  int32_t n_slots;     /* slots per layer cache                                  */
  int32_t max_pos;     /* every position lies in [0, max_pos)                    */
  int32_t n_idx;       /* indexer key heads per late layer, head_dim wide each;
                          0 = none (see rf_fill_opts); 0 .. 8                    */
} rf_shape;

typedef struct rf_plan rf_plan;

/* Create a plan for one shape.  Validates the shape (RF_E_SHAPE / RF_E_ARG).
 * With RF_MAPS_HOST the plan owns two device map buffers of RF_STREAM_GROUP
 * layers each (sized for bf16 maps, or for int8 maps with RF_MAPS_Q8; about
 * 2 x 4 x 52 MB for bf16 maps at d = 5120), one side stream and five events; these
 * are allocated here, on the current device, and released by rf_plan_destroy.
 * Without it the plan allocates nothing on the device. */
rf_status rf_plan_create(const rf_shape* shape, int32_t flags, rf_plan** out);
void rf_plan_destroy(rf_plan* plan);

/* Workspace bytes rf_fill (or rf_fill_q8 for an RF_MAPS_Q8 plan) needs for
 * n_fill rows when `layers_per_launch` late layers are processed per launch
 * (1 .. n_late; larger means fewer, wider launches; at most RF_STREAM_GROUP
 * count for an RF_MAPS_HOST plan, larger values give that figure).  The call uses the widest
 * grouping the given workspace allows, so any size >=
 * rf_fill_workspace_bytes(plan, n_fill, 1) works.  The figure includes the
 * RoPE table built when none is passed, the per-row sums of squares and norm
 * factors of each launch layer's map output and, for RF_MAPS_Q8 plans, the
 * bf16 image of each launch's maps.  Returns 0 for a bad argument. */
size_t rf_fill_workspace_bytes(const rf_plan* plan, int32_t n_fill, int32_t layers_per_launch);

/* Workspace bytes rf_kv_project needs (one prepared [W_k|W_v] copy and one
 * fp32 norm factor per plan row for each layer of a group, plus the RoPE table
 * if none is passed); same grouping rule, except that RF_MAPS_HOST does not
 * cap the group (no maps are involved). */
size_t rf_kv_project_workspace_bytes(const rf_plan* plan, int32_t layers_per_launch);

/* Fill `table` (device, fp32 [max_pos][head_dim/2][2] = (cos, sin)) with the
 * rotation of every position and pair, angles formed in double precision.
 * rf_fill and rf_kv_project accept this table or build it themselves. */
rf_status rf_rope_table(const rf_plan* plan, float* table, void* hip_stream);

/* Section 2.1: the rows the fill writes are all rows minus the exact set.
 *   exact_rows  [n_exact] int32, any order, duplicates allowed, each in [0, n_rows)
 *   fill_rows   [n_rows]  int32 out: the fill rows, ascending, in the first
 *               *n_fill entries (the rest is left untouched)
 *   n_fill      [1] int32 out (device)
 *   workspace   >= rf_fill_rows_workspace_bytes(n_rows) bytes, 256-byte aligned
 * Out-of-range exact rows are ignored. */
size_t rf_fill_rows_workspace_bytes(int32_t n_rows);
rf_status rf_fill_rows(rf_plan* plan, const int32_t* exact_rows, int32_t n_exact,
                       int32_t* fill_rows, int32_t* n_fill,
                       void* workspace, size_t ws_bytes, void* hip_stream);

/* rf_fill_rows for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same fill-row set, same arguments without the workspace.  Its scratch
 * (row mask, block counts and offsets) is a device array owned by the library,
 * sized for RF_NOALLOC_MAX_ROWS rows (about 1 MiB) and held on each GPU the
 * library runs on until the process ends; the call allocates nothing.  Plans
 * with n_rows > RF_NOALLOC_MAX_ROWS get RF_E_SHAPE, before anything is
 * enqueued.  All calls on one GPU share that array: calls ordered on one
 * stream are fine (each call clears what it uses with a kernel, no memset),
 * calls that overlap on one GPU race.  The call is not timed by
 * rf_plan_profile (timing would create events). */
#define RF_NOALLOC_MAX_ROWS (1 << 20)
rf_status rf_fill_rows_noalloc(rf_plan* plan, const int32_t* exact_rows, int32_t n_exact,
                               int32_t* fill_rows, int32_t* n_fill, void* hip_stream);

/* Value rescale applied by the fill (section 2.3, "Value rescale"; see
 * rf_value_scales below).  With a non-NULL rf_vscale, value head h of filled
 * row r in late layer l is multiplied by
 *     scale[(l * n_groups + group_of_row[r]) * n_kv + h]
 * in fp32, together with the norm's factor, before rounding to bf16; keys are
 * not touched.  Rows whose group is outside [0, n_groups) are skipped (not
 * written), like rows with an out-of-range slot.  A NULL rf_vscale, or all
 * scales 1, gives exactly the unscaled bytes. */
typedef struct rf_vscale {
  const float* scale;           /* device fp32 [n_late][n_groups][n_kv], 4-byte aligned */
  const int32_t* group_of_row;  /* device int32 [n_rows]: request (group) of each row    */
  int32_t n_groups;             /* >= 1                                                    */
} rf_vscale;

/* The value-scale measurement (section 2.3, see rf_value_scales below) run
 * inside the fill: each layer group's scales are measured from the
 * calibration rows with the maps the fill has already loaded for that group,
 * written to `scale`, and applied to the group's filled values like an
 * rf_vscale.  Scales and outputs are bitwise those of rf_value_scales followed
 * by rf_fill with an rf_vscale; streamed maps (RF_MAPS_HOST) cross PCIe once.
 *   layer_in     HOST array of n_late device pointers: true input of each
 *                calibration row, bf16 [n_calib][ld_in], 16-byte aligned
 *   calib_rows   device int32 [n_calib]: the calibration rows (rows of x)
 *   calib_group  device int32 [n_calib]: request of each, in [0, n_groups)
 *   group_of_row device int32 [n_rows]: request of every row (for applying)
 *   scale        device fp32 [n_late][n_groups][n_kv], 4-byte aligned; written
 *   workspace    device, >= rf_value_scales_workspace_bytes(plan, n_calib, 1),
 *                256-byte aligned (separate from the fill's workspace) */
typedef struct rf_vmeasure {
  const uint16_t* const* layer_in;
  int64_t ld_in;
  const int32_t* calib_rows;
  const int32_t* calib_group;
  int32_t n_calib;
  const int32_t* group_of_row;
  int32_t n_groups;
  float* scale;
  void* workspace;
  size_t ws_bytes;
} rf_vmeasure;

/* Options of a fill (HOST struct; pass NULL for none of them).
 *   vscale  value rescale (above), or NULL
 *   k_norm  QK-norm for layers that normalise their keys (RidgeFill section
 *           6.6 and section 7: in the Qwen layers queries and keys are
 *           normalised per head ahead of attention): HOST array of n_late device pointers, each bf16
 *           [head_dim], 16-byte aligned; or NULL.  Each key head is divided by
 *           sqrt(mean of its head_dim squares + rms_eps) and multiplied by the
 *           gain per dimension, after the key projection and before RoPE.
 *   w_idx, idx_cache  indexer keys, required exactly when the plan's n_idx > 0
 *           (RidgeFill section 2.1 and section 5.1: in sparse-attention layers
 *           filled rows also write the indexer's keys, one 128-wide key head
 *           shared by the indexer's query heads).  HOST arrays of n_late
 *           device pointers, 16-byte aligned: w_idx bf16 [n_idx*head_dim][d_out]
 *           (the indexer key projection), idx_cache bf16
 *           [n_slots][n_idx*head_dim].  Each indexer head is the normalised
 *           input times W_idx, rotated like the attention keys (same theta and
 *           pairing), without QK-norm; it is stored at the row's slot like K.
 *   measure value-scale measurement inside the fill (rf_vmeasure above), or
 *           NULL; replaces vscale (give at most one of the two); rf_fill and
 *           rf_fill_q8 only.  The measurement runs on a stream of the plan's
 *           own, beside the fill's launches (each layer group's K/V launch
 *           waits for its scales, and the call's work ends on hip_stream as
 *           usual); the first fill that measures creates that stream and two
 *           events, kept until rf_plan_destroy. */
typedef struct rf_fill_opts {
  const rf_vscale* vscale;
  const uint16_t* const* k_norm;
  const uint16_t* const* w_idx;
  uint16_t* const* idx_cache;
  const rf_vmeasure* measure;
} rf_fill_opts;

/* The fill (steps 1-5 above) for n_fill rows and every late layer.
 *   x              [n_rows][ld_x] bf16, ld_x >= d_in, ld_x % 8 == 0, 16-byte aligned
 *   fill_rows      [n_fill] int32, ascending, unique, in [0, n_rows)
 *   positions      [n_rows] int32, RoPE position of each row, in [0, max_pos)
 *   slot_of_row    [n_rows] int32 cache slot of each row in [0, n_slots), or
 *                  NULL for slot = row
 *   map_a, map_b   HOST arrays of n_late pointers to A_l, b_l (device pointers,
 *                  or pinned host pointers with RF_MAPS_HOST; the caller keeps
 *                  pinned maps alive until the stream has completed)
 *   gamma, w_k, w_v, k_cache, v_cache   HOST arrays of n_late device pointers
 *   rope_cos_sin   table from rf_rope_table, or NULL (built in the workspace)
 *   opts           HOST pointer to rf_fill_opts (value rescale, QK-norm), or NULL
 *   workspace      >= rf_fill_workspace_bytes(plan, n_fill, 1), 256-byte aligned
 * Rows whose position or slot is out of range are skipped by the kernels
 * (RF_VALIDATE turns them into RF_E_ROWS).  n_fill == 0 enqueues nothing and
 * leaves every cache byte untouched.  Results do not depend on the grouping
 * of layers per launch or on RF_MAPS_HOST: the outputs are bitwise identical. */
rf_status rf_fill(rf_plan* plan,
                  const uint16_t* x, int64_t ld_x,
                  const int32_t* fill_rows, int32_t n_fill,
                  const int32_t* positions, const int32_t* slot_of_row,
                  const uint16_t* const* map_a, const uint16_t* const* map_b,
                  const uint16_t* const* gamma,
                  const uint16_t* const* w_k, const uint16_t* const* w_v,
                  const float* rope_cos_sin,
                  uint16_t* const* k_cache, uint16_t* const* v_cache,
                  const rf_fill_opts* opts,
                  void* workspace, size_t ws_bytes, void* hip_stream);

/* ---- int8 maps -----------------------------------------------------------
 * Section 2.2 ("Size and cost") and section 4.2: the 27B deployment stores
 * each map as int8 codes with one bf16 scale for each 128-weight block of a row, half
 * the bytes of a bf16 map.  The weight is w[o][k] = q[o][k] * s[o][k / 128]:
 *    map_q      [d_out][d_in] int8 codes, 16-byte aligned
 *    map_scale  [d_out][d_in / 128] bf16 scales
 * rf_fill_q8 is rf_fill for a plan created with RF_MAPS_Q8: before each launch
 * group's map contraction it expands the group's maps into a bf16 image in the
 * workspace, rounding each product q * s once to bf16 (nearest even; the exact
 * product has at most 16 significant bits), and then runs rf_fill's kernels on
 * that image.  Its output is therefore bitwise equal to rf_fill given
 * map_a[l] = rf_map_dequantize_q8(map_q[l], map_scale[l]).  With RF_MAPS_HOST
 * map_q, map_scale and map_b are pinned HOST pointers; the copies move half
 * the bytes of bf16 maps.  Other arguments and rules as for rf_fill.
 * RF_E_ARG if the plan's RF_MAPS_Q8 flag does not match the call. */
rf_status rf_fill_q8(rf_plan* plan,
                     const uint16_t* x, int64_t ld_x,
                     const int32_t* fill_rows, int32_t n_fill,
                     const int32_t* positions, const int32_t* slot_of_row,
                     const int8_t* const* map_q, const uint16_t* const* map_scale,
                     const uint16_t* const* map_b,
                     const uint16_t* const* gamma,
                     const uint16_t* const* w_k, const uint16_t* const* w_v,
                     const float* rope_cos_sin,
                     uint16_t* const* k_cache, uint16_t* const* v_cache,
                     const rf_fill_opts* opts,
                     void* workspace, size_t ws_bytes, void* hip_stream);

/* Expand one int8 map into bf16 (device to device): w[o][k] = bf16(q[o][k] *
 * s[o][k / 128]), nearest even.  d_in % 128 == 0, d_out >= 1; q and w 16-byte
 * aligned.  The kernel rf_fill_q8 runs before each map contraction. */
rf_status rf_map_dequantize_q8(const int8_t* q, const uint16_t* scale, int32_t d_out, int32_t d_in,
                               uint16_t* w, void* hip_stream);

/* Quantize an fp32 map (HOST, [d_out][d_in], d_in % 128 == 0) to the int8
 * format, absmax per 128-weight block: s = bf16 (nearest even) of the fp32
 * value nearest max|a| / 127, q = a / s rounded to nearest (ties to even) in
 * double precision and clipped to [-127, 127]; an all-zero block gets s = 0,
 * q = 0.  Outputs q [d_out][d_in] and scale [d_out][d_in / 128], HOST. */
rf_status rf_map_quantize_q8(const float* a, int32_t d_out, int32_t d_in, int8_t* q, uint16_t* scale);

/* ---- Value rescale measurement --------------------------------------------
 * Section 2.3 ("Value rescale"), on for the 27B deployment with c = 512
 * (section 4.2): in each late layer, the first c rows of each request's tail
 * are projected to values twice, from their true input and from the map's
 * prediction; per request g and key-value head h the scale is the mean over
 * the request's rows of ||v_exact_h|| / ||v_pred_h|| (Euclidean norms over the
 * head's head_dim values).  Rows whose predicted head norm is zero are left
 * out; a (request, head) with no rows gets scale 1.
 *   x              split state, as for rf_fill
 *   layer_in       HOST array of n_late device pointers; layer_in[l] is bf16
 *                  [n_calib][ld_in]: the true input of layer l for each
 *                  calibration row, in calibration order (ld_in >= d_out, % 8)
 *   calib_rows     [n_calib] int32 rows of x (the calibration rows)
 *   calib_group    [n_calib] int32 request of each calibration row
 *   n_groups       requests (>= 1); scale[l][g][h] is written for every g
 *   map_*, gamma, w_v   as for rf_fill / rf_fill_q8 (RF_MAPS_HOST streams)
 *   scale          device fp32 [n_late][n_groups][n_kv] out, 4-byte aligned
 *   workspace      >= rf_value_scales_workspace_bytes(plan, n_calib, 1)
 * Both value vectors go through the fill's own kernels (map contraction, norm
 * and value projection, bf16 rounding); the norms, ratios and means are fp32
 * with a fixed summation order.  The result feeds rf_fill's rf_vscale. */
size_t rf_value_scales_workspace_bytes(const rf_plan* plan, int32_t n_calib, int32_t layers_per_launch);
rf_status rf_value_scales(rf_plan* plan,
                          const uint16_t* x, int64_t ld_x,
                          const uint16_t* const* layer_in, int64_t ld_in,
                          const int32_t* calib_rows, const int32_t* calib_group,
                          int32_t n_calib, int32_t n_groups,
                          const uint16_t* const* map_a, const uint16_t* const* map_b,
                          const uint16_t* const* gamma, const uint16_t* const* w_v,
                          float* scale, void* workspace, size_t ws_bytes, void* hip_stream);
rf_status rf_value_scales_q8(rf_plan* plan,
                             const uint16_t* x, int64_t ld_x,
                             const uint16_t* const* layer_in, int64_t ld_in,
                             const int32_t* calib_rows, const int32_t* calib_group,
                             int32_t n_calib, int32_t n_groups,
                             const int8_t* const* map_q, const uint16_t* const* map_scale,
                             const uint16_t* const* map_b,
                             const uint16_t* const* gamma, const uint16_t* const* w_v,
                             float* scale, void* workspace, size_t ws_bytes, void* hip_stream);

/* The exact cache write of each late layer from given true inputs: steps 2-5
 * only (no map).  Section 2.1: for exact rows and the tail each late layer
 * starts from the input the full model computes; with every layer_in[l] = x
 * and A_l = I, b_l = 0, rf_fill gives
 * the same bytes (the identity fill of section 7, POP's fill).
 *   layer_in   HOST array of n_late device pointers, each bf16 [n_rows][ld_in]
 *              (entries may alias), ld_in >= d_out, ld_in % 8 == 0
 *   rows       [n] int32 rows to write, in [0, n_rows), unique
 *   opts       as for rf_fill, but without a value rescale (RF_E_ARG if
 *              opts->vscale is set): exact rows are not rescaled
 *   other arguments as for rf_fill. */
rf_status rf_kv_project(rf_plan* plan,
                        const uint16_t* const* layer_in, int64_t ld_in,
                        const int32_t* rows, int32_t n,
                        const int32_t* positions, const int32_t* slot_of_row,
                        const uint16_t* const* gamma,
                        const uint16_t* const* w_k, const uint16_t* const* w_v,
                        const float* rope_cos_sin,
                        uint16_t* const* k_cache, uint16_t* const* v_cache,
                        const rf_fill_opts* opts,
                        void* workspace, size_t ws_bytes, void* hip_stream);

/* ---- Closed-form ridge map, HOST memory, float64 inside (validation only) ----
 * Section 2.2: with X and Y centred, A = Y^T X (X^T X + alpha I)^(-1) and
 * b = mu_Y - A mu_X, alpha = lambda * tr(Xc^T Xc) / d_in; only A is penalised.
 * "Fitting": X^T X, X^T Y and the means, summed over documents, lead to the
 * same maps as one solve; a different lambda costs one more solve, not a pass.
 * X is [n][d_in] fp32, Y is [n][d_out] fp32 (row-major, HOST).  Products are
 * formed and summed in float64.  A is returned [d_out][d_in] (the layout
 * rf_fill's map_a takes) and b [d_out], both fp32 HOST. */
typedef struct rf_ridge_acc rf_ridge_acc;
rf_status rf_ridge_acc_create(int32_t d_in, int32_t d_out, rf_ridge_acc** out);
rf_status rf_ridge_acc_add(rf_ridge_acc* acc, const float* x, const float* y, int64_t n);
rf_status rf_ridge_solve(const rf_ridge_acc* acc, double lambda, int32_t flags,
                         float* a, float* b);
void rf_ridge_acc_destroy(rf_ridge_acc* acc);
/* The running sums themselves (HOST, fp64; any output pointer may be NULL):
 * sxx [d_in][d_in] (full, symmetric), sxy [d_in][d_out], sx [d_in], sy [d_out], n. */
rf_status rf_ridge_acc_sums(const rf_ridge_acc* acc, double* sxx, double* sxy, double* sx, double* sy, int64_t* n);
/* create + add + solve + destroy in one call */
rf_status rf_ridge_fit(const float* x, const float* y, int64_t n, int32_t d_in, int32_t d_out,
                       double lambda, int32_t flags, float* a, float* b);

/* ---- Device capture of the ridge sums --------------------------------------
 * Section 2.2 ("Fitting"): the running sums of X^T X, X^T Y, X and Y that the
 * ridge solve needs, formed on the GPU from calibration activations that are
 * already there (bf16 split states X [n][ld_x] and layer inputs Y [n][ld_y],
 * device memory, 16-byte aligned, ld multiples of 8).  bf16 values and their
 * products are exact in fp64, and the sums are accumulated in fp64 with
 * matrix instructions, so they equal rf_ridge_acc_add's on the same values up
 * to the order of the fp64 additions.  X^T X is formed on its upper tiles only.
 *   create   d_in, d_out positive multiples of 128; allocates the sums
 *            ((d_in + d_out) * d_in + 64 * max(d_in, d_out) + d_in + d_out
 *            doubles) on the current device and zeroes them (synchronously)
 *   add      enqueues on hip_stream; n == 0 is a no-op
 *   merge    waits for hip_stream, adds the sums into a host accumulator of
 *            the same d_in, d_out, and clears them; then rf_ridge_solve */
typedef struct rf_ridge_dev rf_ridge_dev;
rf_status rf_ridge_dev_create(int32_t d_in, int32_t d_out, rf_ridge_dev** out);
rf_status rf_ridge_dev_add(rf_ridge_dev* dev, const uint16_t* x, int64_t ld_x, const uint16_t* y, int64_t ld_y,
                           int64_t n, void* hip_stream);
rf_status rf_ridge_dev_merge(rf_ridge_dev* dev, rf_ridge_acc* acc, void* hip_stream);
void rf_ridge_dev_destroy(rf_ridge_dev* dev);

/* The ridge solve of section 2.2 on the GPU, from the device sums (which it
 * leaves unchanged, so another lambda needs only another solve).  Same
 * definition and flags as rf_ridge_solve: centred sums, alpha = lambda *
 * tr(Xc^T Xc) / d_in, A = Y^T X (X^T X + alpha I)^(-1), b = mu_Y - A mu_X (with
 * RF_RIDGE_RAW: no centring, alpha = lambda, b = 0), in fp64 with a blocked
 * Cholesky factorisation and triangular solves; results are bitwise
 * reproducible.  Outputs are DEVICE fp32, 4-byte aligned: a [d_out][d_in] (the
 * layout rf_fill's map_a takes, after rounding to bf16), b [d_out].  The
 * workspace (256-byte aligned, rf_ridge_dev_solve_workspace_bytes) holds the
 * factor and the right-hand sides in fp64.  The call synchronises hip_stream
 * before it returns, to report a system that is not positive definite
 * (RF_E_LINALG; a and b then hold no meaningful values).  Needs n >= 1. */
size_t rf_ridge_dev_solve_workspace_bytes(const rf_ridge_dev* dev);
rf_status rf_ridge_dev_solve(const rf_ridge_dev* dev, double lambda, int32_t flags, float* a, float* b,
                             void* workspace, size_t ws_bytes, void* hip_stream);

/* ---- Kernel timing -------------------------------------------------------
 * With profiling on, every launch and map copy the plan issues is bracketed
 * by a pair of HIP events recorded on the stream it runs on (the caller's
 * stream, or the side stream for map copies).  rf_plan_profile_read waits for
 * the recorded events, adds up their elapsed times per kind and clears them.
 * Turning profiling on or off discards unread records. */
enum {
  RF_K_MAP = 0,       /* map contraction (map_gemm)                  */
  RF_K_KV = 1,        /* norm + K/V contraction with RoPE and scatter */
  RF_K_PREP = 2,      /* gamma folded into [W_k|W_v]                 */
  RF_K_ROPE = 3,      /* RoPE table                                  */
  RF_K_ROWS = 4,      /* fill-row compaction                         */
  RF_K_COPY = 5,      /* host -> device map copy (RF_MAPS_HOST)      */
  RF_K_DEQUANT = 6,   /* int8 map -> bf16 image (RF_MAPS_Q8)         */
  RF_K_SCALE = 7,     /* every launch of rf_value_scales(_q8) except
                         the int8 expansion (kind RF_K_DEQUANT)      */
  RF_K_NORM = 8,      /* per-row norm factors from the map's row sums */
  RF_K_COUNT = 9
};
typedef struct rf_profile {
  double ms[RF_K_COUNT];        /* summed event time per kind, milliseconds */
  int64_t launches[RF_K_COUNT]; /* launches (or copies) per kind            */
} rf_profile;
rf_status rf_plan_profile(rf_plan* plan, int32_t enable);
rf_status rf_plan_profile_read(rf_plan* plan, rf_profile* out);

/* Thread-local message for the last non-OK status of this thread ("" if none). */
const char* rf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RF_H */
