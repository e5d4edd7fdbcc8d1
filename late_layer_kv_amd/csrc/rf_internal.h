// Internal interface between the host API (rf_api.cpp) and the kernels
// (rf_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rf {

// Layers handled by one launch (kernel arguments carry per-layer pointers).
constexpr int kMaxGroup = 32;
// Macro tile of both contractions: 256 output features x 256 rows, 64-deep
// contraction steps.
constexpr int kTileN = 256;
constexpr int kTileM = 256;
constexpr int kTileK = 64;

// Map contraction, section 2.2 of the paper: Y_g[m][n] = bf16(sum_k A_g[n][k] x[row(m)][k] + b_g[n]).
struct MapParams {
  const uint16_t* x;      // [n_rows][ld_x]
  int64_t ld_x;
  const int32_t* rows;    // [M] gather index into x
  int32_t n_rows;
  int32_t M;              // rows of this call (n_fill)
  int32_t K;              // d_in
  int32_t N;              // d_out
  int32_t tiles_m, tiles_n;
  uint16_t* y;            // [n_layers][M][N]
  // Row sums of squares of the stored (bf16) Y, one partial per 256-feature
  // tile: ssq[(g * tiles_n + tn) * M + m], or null (not written).
  float* ssq;
  const uint16_t* a[kMaxGroup];  // [N][K]
  const uint16_t* b[kMaxGroup];  // [N]
};

// Norm + key/value contraction with the RoPE and cache-scatter epilogue:
//   acc[m][f] = sum_k in_g[src(m)][k] * Wp_g[f][k],  Wp_g = bf16(W_kv * gamma)
//   out = acc * rs_g[m], RoPE on key features, bf16 to the cache, where
//   rs_g[m] = 1 / sqrt(mean_k in_g[src(m)][k]^2 + eps) comes precomputed
//   (launch_row_scale from the map's row sums, or launch_row_rms).
struct KvParams {
  int64_t ld_in;
  const int32_t* in_rows;   // [M] gather index into in_g, or null (row m)
  int32_t n_in_rows;        // rows addressable in in_g
  const int32_t* out_rows;  // [M] global row id of m (positions/slots), or null
  int32_t M;
  int32_t K;                // d_out (normalised width)
  int32_t w;                // n_kv * head_dim
  int32_t widx;             // indexer key columns (n_idx * head_dim), after the values
  int32_t head_dim;
  int32_t tiles_m, tiles_n;
  int32_t group_m;          // row tiles per group of the tile order (set by launch_kv)
  // Indexer remainder: >= 0, the first of 128 features (prepared-weight rows)
  // that tall tiles of 512 rows compute (tiles_n then stops short of them);
  // -1: none.  Value-only launches ignore it.
  int32_t tall_f0;
  int32_t wrows;            // rows per layer of wkv: 2w + widx rounded up to 256
  const uint16_t* wkv;      // [n_layers][wrows][K] prepared weights (zero rows past 2w + widx)
  const int32_t* positions; // [n_rows]
  const int32_t* slots;     // [n_rows] or null (slot = row)
  int32_t n_rows, n_slots, max_pos;
  const float* rope;        // [max_pos][head_dim/2][2]
  float eps;
  // Value rescale (when group_of_row is set; then every vscale[g] of the launch
  // must be set): value head h of row r is multiplied by
  // vscale_g[group_of_row[r] * n_kv + h] before rounding.  Rows whose group is
  // outside [0, n_groups) are skipped like bad slots.
  const int32_t* group_of_row;  // [n_rows] or null
  int32_t n_groups, n_kv;
  // v_only: tiles start at the 256-feature tile holding feature w (tiles_n =
  // (2w - that offset) / 256); only value features are stored, keys are
  // neither rotated nor written (kc may be null).
  int32_t v_only;
  // QK-norm: each key head is divided by sqrt(mean of its squares + eps) and
  // multiplied by kgamma_g[j] (bf16 [head_dim]) before RoPE.
  int32_t qk_norm;
  const uint16_t* in[kMaxGroup];
  uint16_t* kc[kMaxGroup];  // [n_slots][w]
  uint16_t* vc[kMaxGroup];
  uint16_t* ic[kMaxGroup];  // [n_slots][widx] indexer keys (widx > 0)
  const float* vscale[kMaxGroup];  // [n_groups][n_kv] per layer, or null
  const uint16_t* kgamma[kMaxGroup];  // [head_dim] per layer (qk_norm)
  const float* rs[kMaxGroup];  // [M] norm factor of row m of this call, per layer
};

// Prepared projection weights: out_g[f][k] = bf16(W[f][k] * gamma_g[k]),
// W = W_k for f < w, W_v (row f - w) for f < 2w, W_idx (row f - 2w) for
// f < 2w + widx, zero up to rows.
struct PrepParams {
  int32_t d;       // d_out
  int32_t w;
  int32_t widx;
  int32_t rows;    // rows per layer, >= 2w + widx
  uint16_t* out;   // [n_layers][rows][d]
  const uint16_t* gamma[kMaxGroup];
  const uint16_t* wk[kMaxGroup];
  const uint16_t* wv[kMaxGroup];
  const uint16_t* wi[kMaxGroup];
};

// int8 map -> bf16 image: w_g[o][k] = bf16(q_g[o][k] * s_g[o][k / 128]), nearest even.
constexpr int kQ8Block = 128;
struct DequantParams {
  int32_t d_out, d_in;
  const int8_t* q[kMaxGroup];     // [d_out][d_in]
  const uint16_t* s[kMaxGroup];   // [d_out][d_in / 128]
  uint16_t* w[kMaxGroup];         // [d_out][d_in]
};

hipError_t launch_map(const MapParams& p, int n_layers, hipStream_t s);
// rs[g * M + m] = 1 / sqrt(sum_t ssq[(g * tiles + t) * M + m] * inv_k + eps), the
// map's tile partials summed in tile order.
hipError_t launch_row_scale(const float* ssq, int tiles, int M, int n_layers, float inv_k, float eps, float* rs,
                            hipStream_t s);
hipError_t launch_dequant(const DequantParams& p, int n_layers, hipStream_t s);

// Value-rescale measurement: per layer, ratio[m][h] = ||ve[m][h]|| / ||vp[m][h]|| over the
// head's hd values (-1 when the predicted norm is zero), then per (layer, group, head)
// the mean of the non-negative ratios of the rows of that group, in row order (1 if none).
struct RatioParams {
  int32_t n, n_kv, head_dim;
  const uint16_t* ve[kMaxGroup];  // [n][n_kv * head_dim]
  const uint16_t* vp[kMaxGroup];
  float* ratio[kMaxGroup];        // [n][n_kv]
};
hipError_t launch_head_ratio(const RatioParams& p, int n_layers, hipStream_t s);
// p[0..n) = 0 (a fill kernel: no memset node if the caller captures the stream)
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
// ratio [n_late][n][n_kv] -> scale [n_late][n_groups][n_kv]
hipError_t launch_scale_mean(const float* ratio, const int32_t* group, int n, int n_kv, int n_groups,
                             int n_late, float* scale, hipStream_t s);
hipError_t launch_kv(const KvParams& p, int n_layers, hipStream_t s);
// rs[g * M + m] = 1 / sqrt(mean_k in_g[src(m)][k]^2 + eps) for inputs that do
// not come from the map contraction (src as in KvParams).
struct RmsParams {
  int64_t ld_in;
  const int32_t* in_rows;  // [M] or null (row m)
  int32_t n_in_rows, M, K;  // K a multiple of 256
  float inv_k, eps;        // inv_k = 1.0f / K, as the map path's row_scale is given it
  float* rs;               // [n_layers][M]
  const uint16_t* in[kMaxGroup];
};
hipError_t launch_row_rms(const RmsParams& p, int n_layers, hipStream_t s);
hipError_t launch_prep(const PrepParams& p, int n_layers, hipStream_t s);
hipError_t launch_rope_table(float* table, int max_pos, int head_dim, double theta, hipStream_t s);
// The fill-row set (rf_rows.hip): fill_rows = ascending rows of [0, n_rows)
// not in exact, *n_fill their count.  ws holds fill_rows_ws_bytes(n_rows)
// bytes, 256-byte aligned.
size_t fill_rows_ws_bytes(int n_rows);
hipError_t launch_fill_rows(const int32_t* exact, int n_exact, int n_rows, void* ws, int32_t* fill_rows,
                            int32_t* n_fill, hipStream_t s);
// Largest batch the library takes (row indices and the padded row mask stay in int).
constexpr int kMaxRows = 1 << 30;
// The same with the library's own scratch array (no workspace): at most
// kNoAllocMaxRows rows (RF_NOALLOC_MAX_ROWS in rf.h).
constexpr int kNoAllocMaxRows = 1 << 20;
hipError_t launch_fill_rows_noalloc(const int32_t* exact, int n_exact, int n_rows, int32_t* fill_rows,
                                    int32_t* n_fill, hipStream_t s);
// Sets bits in *flag: 1 row out of range, 2 position out of range,
// 4 slot out of range, 8 rows not strictly ascending.
hipError_t launch_validate(const int32_t* rows, int n, int n_rows, int ascending,
                           const int32_t* positions, int max_pos, const int32_t* slots,
                           int n_slots, int32_t* flag, hipStream_t s);

}  // namespace rf
