// Host side of the C ABI in include/rf.h: argument checks, workspace layout,
// layer grouping, and the pipeline that streams host-resident maps.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <memory>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/rf.h"
#include "rf_error.h"
#include "rf_internal.h"

namespace {

thread_local std::string g_err;

rf_status fail(rf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

rf_status hip_fail(hipError_t e, const char* what) {
  return fail(RF_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

void rf::set_last_error(const char* msg) { g_err = msg; }

struct rf_plan {
  rf_shape s{};
  int32_t flags = 0;
  // The value-scale measurement inside a fill runs on its own stream, beside
  // the fill's launches: to_meas orders it after the fill's stream, from_meas
  // the other way.  Created by the first fill that measures.
  hipStream_t meas = nullptr;
  hipEvent_t to_meas = nullptr, from_meas = nullptr;
  hipError_t make_meas_stream() {
    if (meas) return hipSuccess;
    hipError_t e = hipEventCreateWithFlags(&to_meas, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&from_meas, hipEventDisableTiming);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&meas, hipStreamNonBlocking);
    return e;
  }
  // RF_MAPS_HOST only
  hipStream_t side = nullptr;
  hipEvent_t ev_start = nullptr;
  hipEvent_t ev_copied[2] = {nullptr, nullptr};
  hipEvent_t ev_consumed[2] = {nullptr, nullptr};
  // Up to RF_STREAM_GROUP streamed layers per buffer, layer_bytes apart, each
  // the map (bf16 [d_out][d_in], or int8 codes [d_out][d_in] then bf16 scales
  // [d_out][d_in/128]) and then b [d_out].
  char* mapbuf[2] = {nullptr, nullptr};
  size_t map_bytes = 0;    // bf16 map, or int8 codes
  size_t scale_off = 0;    // byte offset of the scales (int8 maps)
  size_t scale_bytes = 0;
  size_t bias_off = 0;     // byte offset of b
  size_t layer_bytes = 0;  // one layer's part of a buffer
  // kernel timing (rf_plan_profile)
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  bool prof = false;
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t take_event() {
    hipEvent_t e = nullptr;
    if (!pool.empty()) {
      e = pool.back();
      pool.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
    }
    return e;
  }
  void drop_records() {
    for (auto& r : recs) {
      pool.push_back(r.a);
      pool.push_back(r.b);
    }
    recs.clear();
  }
};

namespace {

// Brackets one launch (or copy) with an event pair when profiling is on.
class Timed {
 public:
  Timed(rf_plan* p, int kind, hipStream_t s) : p_(p), kind_(kind), s_(s) {
    if (p_ && p_->prof && (a_ = p_->take_event())) (void)hipEventRecord(a_, s_);
  }
  ~Timed() {
    if (!a_) return;
    hipEvent_t b = p_->take_event();
    if (b && hipEventRecord(b, s_) == hipSuccess) {
      p_->recs.push_back({kind_, a_, b});
    } else {
      p_->pool.push_back(a_);
      if (b) p_->pool.push_back(b);
    }
  }

 private:
  rf_plan* p_;
  int kind_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr;
};

}  // namespace

namespace {

int kv_width(const rf_shape& s) { return s.n_kv * s.head_dim; }
int idx_width(const rf_shape& s) { return s.n_idx * s.head_dim; }
// prepared-weight rows per layer: keys, values, indexer keys, zero rows up to a whole tile
int prep_rows(const rf_shape& s) { return (2 * kv_width(s) + idx_width(s) + rf::kTileN - 1) / rf::kTileN * rf::kTileN; }
// Indexer key columns ending half way into a 256-feature tile (a 128-wide
// remainder) go to tall tiles of the K/V launch (512 rows x 128 features)
// instead of a tile that is half zero padding, when every layer input and the
// layer's prepared weights span less than 4 GiB (those tiles' loads use 32-bit
// offsets).  Returns the first feature of the remainder, or -1 to let the K/V
// kernel cover every column.
int tall_f0(const rf_shape& s, int64_t in_rows, int64_t ld_in) {
  const int cols = 2 * s.n_kv * s.head_dim + s.n_idx * s.head_dim;
  if (s.n_idx == 0 || cols % rf::kTileN != 128) return -1;
  const int64_t limit = int64_t(1) << 32;
  if (in_rows * ld_in * 2 >= limit || int64_t(prep_rows(s)) * s.d_out * 2 >= limit) return -1;
  return cols - 128;
}
size_t rope_bytes(const rf_shape& s) { return up(static_cast<size_t>(s.max_pos) * (s.head_dim / 2) * 8); }
size_t prep_bytes(const rf_shape& s, int g) {
  return up(static_cast<size_t>(g) * prep_rows(s) * s.d_out * 2);
}
size_t y_bytes(const rf_shape& s, int n_fill, int g) {
  return up(static_cast<size_t>(g) * n_fill * s.d_out * 2);
}
// Per-row norm of each launch layer's Y: the map's per-tile sums of squares,
// then the factor 1 / sqrt(mean + eps) per row.
size_t ssq_bytes(const rf_shape& s, int n_fill, int g) {
  return up(static_cast<size_t>(g) * (s.d_out / rf::kTileN) * n_fill * 4);
}
size_t rs_bytes(int n_fill, int g) { return up(static_cast<size_t>(g) * n_fill * 4); }
// bf16 image of the int8 maps of one launch group (RF_MAPS_Q8 plans only)
size_t dq_bytes(const rf_shape& s, int32_t flags, int g) {
  return (flags & RF_MAPS_Q8) ? up(static_cast<size_t>(g) * s.d_out * s.d_in * 2) : 0;
}
constexpr size_t kFlagBytes = kAlign;

rf_status check_shape(const rf_shape* s, int32_t flags) {
  if (!s) return fail(RF_E_ARG, "shape is null");
  if (flags & ~(RF_MAPS_HOST | RF_VALIDATE | RF_MAPS_Q8)) return fail(RF_E_ARG, "unknown flag bits 0x%x", flags);
  if ((flags & RF_MAPS_Q8) && s->d_in % rf::kQ8Block)
    return fail(RF_E_SHAPE, "d_in=%d must be a multiple of %d for int8 maps", s->d_in, rf::kQ8Block);
  if (s->d_in <= 0 || s->d_in % rf::kTileK)
    return fail(RF_E_SHAPE, "d_in=%d must be a positive multiple of %d", s->d_in, rf::kTileK);
  if (s->d_out <= 0 || s->d_out % rf::kTileN)
    return fail(RF_E_SHAPE, "d_out=%d must be a positive multiple of %d", s->d_out, rf::kTileN);
  if (s->n_late < 1) return fail(RF_E_SHAPE, "n_late=%d must be >= 1", s->n_late);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(RF_E_SHAPE, "head_dim=%d must be 64 or 128", s->head_dim);
  if (s->n_kv < 1 || (s->n_kv * s->head_dim) % 128)
    return fail(RF_E_SHAPE, "n_kv*head_dim=%d must be a positive multiple of 128", s->n_kv * s->head_dim);
  if (!(s->rms_eps >= 0.0f)) return fail(RF_E_SHAPE, "rms_eps must be >= 0");
  if (!(s->rope_theta > 1.0)) return fail(RF_E_SHAPE, "rope_theta must be > 1");
  if (s->n_rows < 0 || s->n_slots < 0 || s->max_pos < 1)
    return fail(RF_E_SHAPE, "n_rows, n_slots must be >= 0 and max_pos >= 1");
  if (s->n_rows > rf::kMaxRows) return fail(RF_E_SHAPE, "n_rows=%d above the limit %d", s->n_rows, rf::kMaxRows);
  if (s->n_idx < 0 || s->n_idx > 8) return fail(RF_E_SHAPE, "n_idx=%d must be in [0, 8]", s->n_idx);
  return RF_OK;
}

// Most layers one launch with maps takes: kMaxGroup, or RF_STREAM_GROUP for
// streamed maps (the plan's map buffers hold that many layers).
int max_group(const rf_plan* p) {
  return std::min(p->s.n_late, (p->flags & RF_MAPS_HOST) ? RF_STREAM_GROUP : rf::kMaxGroup);
}

// Layers in the launch group that starts at layer l0 when groups of up to G
// are allowed.  Streamed maps start with a group of one layer, so that only
// one layer's copy precedes the first launch; later copies overlap the
// previous group's kernels.
int group_at(const rf_plan* p, int l0, int G) {
  if ((p->flags & RF_MAPS_HOST) && l0 == 0) return 1;
  return std::min(G, p->s.n_late - l0);
}

rf_status check_layer_ptrs(const void* const* arr, int n, const char* name, bool need16 = true) {
  if (!arr) return fail(RF_E_ARG, "%s array is null", name);
  for (int i = 0; i < n; ++i) {
    if (!arr[i]) return fail(RF_E_ARG, "%s[%d] is null", name, i);
    if (need16 && !aligned16(arr[i])) return fail(RF_E_ARG, "%s[%d] is not 16-byte aligned", name, i);
  }
  return RF_OK;
}

rf_status run_validate(rf_plan* p, const int32_t* rows, int n, int ascending, const int32_t* positions,
                       const int32_t* slots, int32_t* flag_dev, hipStream_t st) {
  hipError_t e = rf::launch_validate(rows, n, p->s.n_rows, ascending, positions, p->s.max_pos, slots,
                                     p->s.n_slots, flag_dev, st);
  if (e != hipSuccess) return hip_fail(e, "validate launch");
  int32_t flag = 0;
  e = hipMemcpyAsync(&flag, flag_dev, sizeof flag, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "validate readback");
  if (flag)
    return fail(RF_E_ROWS, "row check failed (bits 0x%x: 1 row range, 2 position range, 4 slot range, 8 order)",
                flag);
  return RF_OK;
}

}  // namespace

extern "C" {

const char* rf_last_error(void) { return g_err.c_str(); }

rf_status rf_plan_create(const rf_shape* shape, int32_t flags, rf_plan** out) {
  if (!out) return fail(RF_E_ARG, "out is null");
  *out = nullptr;
  rf_status st = check_shape(shape, flags);
  if (st != RF_OK) return st;
  rf_plan* p = new rf_plan();
  p->s = *shape;
  p->flags = flags;
  hipError_t e = hipSuccess;
  if (flags & RF_MAPS_HOST) {
    const size_t elems = static_cast<size_t>(shape->d_out) * shape->d_in;
    if (flags & RF_MAPS_Q8) {
      p->map_bytes = elems;
      p->scale_off = up(p->map_bytes);
      p->scale_bytes = static_cast<size_t>(shape->d_out) * (shape->d_in / rf::kQ8Block) * 2;
      p->bias_off = p->scale_off + up(p->scale_bytes);
    } else {
      p->map_bytes = elems * 2;
      p->bias_off = up(p->map_bytes);
    }
    p->layer_bytes = up(p->bias_off + static_cast<size_t>(shape->d_out) * 2);
    const size_t bytes = p->layer_bytes * RF_STREAM_GROUP;
    for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipMalloc(reinterpret_cast<void**>(&p->mapbuf[i]), bytes);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&p->side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ev_start, hipEventDisableTiming);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&p->ev_copied[i], hipEventDisableTiming);
    for (int i = 0; i < 2 && e == hipSuccess; ++i)
      e = hipEventCreateWithFlags(&p->ev_consumed[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      rf_plan_destroy(p);
      return hip_fail(e, "plan resources for streamed maps");
    }
  }
  *out = p;
  return RF_OK;
}

void rf_plan_destroy(rf_plan* p) {
  if (!p) return;
  if (p->meas) (void)hipStreamSynchronize(p->meas);
  if (p->to_meas) (void)hipEventDestroy(p->to_meas);
  if (p->from_meas) (void)hipEventDestroy(p->from_meas);
  if (p->meas) (void)hipStreamDestroy(p->meas);
  if (p->side) (void)hipStreamSynchronize(p->side);
  for (int i = 0; i < 2; ++i) {
    if (p->mapbuf[i]) (void)hipFree(p->mapbuf[i]);
    if (p->ev_copied[i]) (void)hipEventDestroy(p->ev_copied[i]);
    if (p->ev_consumed[i]) (void)hipEventDestroy(p->ev_consumed[i]);
  }
  if (p->ev_start) (void)hipEventDestroy(p->ev_start);
  if (p->side) (void)hipStreamDestroy(p->side);
  p->drop_records();
  for (hipEvent_t e : p->pool) (void)hipEventDestroy(e);
  delete p;
}

rf_status rf_plan_profile(rf_plan* p, int32_t enable) {
  if (!p) return fail(RF_E_ARG, "plan is null");
  p->drop_records();
  p->prof = enable != 0;
  return RF_OK;
}

rf_status rf_plan_profile_read(rf_plan* p, rf_profile* out) {
  if (!p || !out) return fail(RF_E_ARG, "null argument");
  *out = rf_profile{};
  for (const auto& r : p->recs) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) {
      p->drop_records();
      return hip_fail(e, "profile read");
    }
    out->ms[r.kind] += ms;
    out->launches[r.kind] += 1;
  }
  p->drop_records();
  return RF_OK;
}

size_t rf_fill_workspace_bytes(const rf_plan* p, int32_t n_fill, int32_t g) {
  if (!p || n_fill < 0 || g < 1 || g > p->s.n_late) return 0;
  g = std::min(g, max_group(p));
  return rope_bytes(p->s) + kFlagBytes + prep_bytes(p->s, g) + y_bytes(p->s, n_fill, g) + dq_bytes(p->s, p->flags, g) +
         ssq_bytes(p->s, n_fill, g) + rs_bytes(n_fill, g);
}

size_t rf_kv_project_workspace_bytes(const rf_plan* p, int32_t g) {
  if (!p || g < 1 || g > p->s.n_late) return 0;
  g = std::min(g, rf::kMaxGroup);
  return rope_bytes(p->s) + kFlagBytes + prep_bytes(p->s, g) + rs_bytes(p->s.n_rows, g);
}

size_t rf_fill_rows_workspace_bytes(int32_t n_rows) {
  if (n_rows < 0 || n_rows > rf::kMaxRows) return 0;
  return rf::fill_rows_ws_bytes(n_rows);
}

rf_status rf_rope_table(const rf_plan* p, float* table, void* stream) {
  if (!p || !table) return fail(RF_E_ARG, "null plan or table");
  if (!aligned16(table)) return fail(RF_E_ARG, "table must be 16-byte aligned");
  hipError_t e = rf::launch_rope_table(table, p->s.max_pos, p->s.head_dim, p->s.rope_theta,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RF_OK : hip_fail(e, "rope table launch");
}

rf_status rf_fill_rows(rf_plan* p, const int32_t* exact_rows, int32_t n_exact, int32_t* fill_rows,
                       int32_t* n_fill, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return fail(RF_E_ARG, "plan is null");
  if (n_exact < 0 || (n_exact > 0 && !exact_rows)) return fail(RF_E_ARG, "bad exact rows");
  if (!fill_rows || !n_fill) return fail(RF_E_ARG, "null output");
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign) || ws_bytes < rf_fill_rows_workspace_bytes(p->s.n_rows))
    return fail(RF_E_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned",
                rf_fill_rows_workspace_bytes(p->s.n_rows));
  Timed tm(p, RF_K_ROWS, static_cast<hipStream_t>(stream));
  hipError_t e = rf::launch_fill_rows(exact_rows, n_exact, p->s.n_rows, ws, fill_rows, n_fill,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RF_OK : hip_fail(e, "fill-row launch");
}

rf_status rf_fill_rows_noalloc(rf_plan* p, const int32_t* exact_rows, int32_t n_exact, int32_t* fill_rows,
                               int32_t* n_fill, void* stream) {
  static_assert(RF_NOALLOC_MAX_ROWS == rf::kNoAllocMaxRows, "header and library agree on the limit");
  if (!p) return fail(RF_E_ARG, "plan is null");
  if (n_exact < 0 || (n_exact > 0 && !exact_rows)) return fail(RF_E_ARG, "bad exact rows");
  if (!fill_rows || !n_fill) return fail(RF_E_ARG, "null output");
  if (p->s.n_rows > RF_NOALLOC_MAX_ROWS)
    return fail(RF_E_SHAPE, "rf_fill_rows_noalloc takes at most %d rows (plan has %d); use rf_fill_rows",
                RF_NOALLOC_MAX_ROWS, p->s.n_rows);
  // (no Timed bracket: with profiling on it may create events, and this entry
  // point allocates nothing in any mode)
  hipError_t e = rf::launch_fill_rows_noalloc(exact_rows, n_exact, p->s.n_rows, fill_rows, n_fill,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RF_OK : hip_fail(e, "fill-row launch (library scratch)");
}

}  // extern "C"

namespace {

// Where a call's maps come from: bf16 matrices, or int8 codes with bf16 block scales.
struct MapSrc {
  const uint16_t* const* a = nullptr;      // bf16 [d_out][d_in]
  const int8_t* const* q = nullptr;        // int8 [d_out][d_in]
  const uint16_t* const* scale = nullptr;  // bf16 [d_out][d_in/128]
  const uint16_t* const* b = nullptr;      // bf16 [d_out]
};

rf_status check_maps(const rf_plan* p, const char* fn, const MapSrc& maps) {
  const int L = p->s.n_late;
  const bool q8 = p->flags & RF_MAPS_Q8;
  const bool host_maps = p->flags & RF_MAPS_HOST;
  if (q8 != (maps.q != nullptr || maps.scale != nullptr))
    return fail(RF_E_ARG, "%s: plan %s RF_MAPS_Q8 (int8 maps go to the _q8 entry points, bf16 maps to the others)",
                fn, q8 ? "has" : "lacks");
  rf_status st;
  if (q8) {
    if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(maps.q), L, "map_q", !host_maps)) != RF_OK) return st;
    if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(maps.scale), L, "map_scale", false)) != RF_OK)
      return st;
  } else if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(maps.a), L, "map_a", !host_maps)) != RF_OK) {
    return st;
  }
  return check_layer_ptrs(reinterpret_cast<const void* const*>(maps.b), L, "map_b", !host_maps);
}

// Hands the map kernel device bf16 maps, one launch group at a time.  Resident
// bf16 maps are used as given; resident int8 maps are expanded into the image
// `dq` first; streamed maps (RF_MAPS_HOST) go through the plan's two device
// buffers on the side stream, alternately, up to RF_STREAM_GROUP layers per
// group: the copy of group j waits until the kernels of group j-2 (same
// buffer) that read the maps have run, and the kernels of group j wait for
// its copy.  The first copies also wait for the work already on the caller's
// stream, which may still read the buffers.
class MapFeeder {
 public:
  MapFeeder(rf_plan* p, const MapSrc& maps, uint16_t* dq, hipStream_t hs)
      : p_(p), maps_(maps), dq_(dq), hs_(hs), q8_(p->flags & RF_MAPS_Q8), host_(p->flags & RF_MAPS_HOST) {
    dp_.d_out = p->s.d_out;
    dp_.d_in = p->s.d_in;
  }
  bool streamed() const { return host_; }

  rf_status begin() {
    if (!host_) return RF_OK;
    hipError_t e;
    if ((e = hipEventRecord(p_->ev_start, hs_)) != hipSuccess) return hip_fail(e, "event record");
    if ((e = hipStreamWaitEvent(p_->side, p_->ev_start, 0)) != hipSuccess) return hip_fail(e, "stream wait");
    return RF_OK;
  }

  // Points mp.a[0..g) and mp.b[0..g) at device bf16 maps of layers l0 .. l0+g-1.
  rf_status load(int l0, int g, rf::MapParams& mp) {
    const size_t elems = static_cast<size_t>(p_->s.d_out) * p_->s.d_in;
    hipError_t e;
    if (!host_) {
      for (int i = 0; i < g; ++i) {
        if (q8_) {
          dp_.q[i] = maps_.q[l0 + i];
          dp_.s[i] = maps_.scale[l0 + i];
          dp_.w[i] = dq_ + i * elems;
          mp.a[i] = dq_ + i * elems;
        } else {
          mp.a[i] = maps_.a[l0 + i];
        }
        mp.b[i] = maps_.b[l0 + i];
      }
      if (q8_) {
        Timed tm(p_, RF_K_DEQUANT, hs_);
        if ((e = rf::launch_dequant(dp_, g, hs_)) != hipSuccess) return hip_fail(e, "dequant launch");
      }
      return RF_OK;
    }
    const int buf = calls_ & 1;
    char* mb = p_->mapbuf[buf];
    if (calls_ >= 2 && (e = hipStreamWaitEvent(p_->side, p_->ev_consumed[buf], 0)) != hipSuccess)
      return hip_fail(e, "stream wait");
    {
      Timed tm(p_, RF_K_COPY, p_->side);
      e = hipSuccess;
      for (int i = 0; i < g && e == hipSuccess; ++i) {
        const int l = l0 + i;
        char* dst = mb + i * p_->layer_bytes;
        const void* msrc = q8_ ? static_cast<const void*>(maps_.q[l]) : static_cast<const void*>(maps_.a[l]);
        e = hipMemcpyAsync(dst, msrc, p_->map_bytes, hipMemcpyHostToDevice, p_->side);
        if (e == hipSuccess && q8_)
          e = hipMemcpyAsync(dst + p_->scale_off, maps_.scale[l], p_->scale_bytes, hipMemcpyHostToDevice, p_->side);
        if (e == hipSuccess)
          e = hipMemcpyAsync(dst + p_->bias_off, maps_.b[l], static_cast<size_t>(p_->s.d_out) * 2,
                             hipMemcpyHostToDevice, p_->side);
      }
      if (e != hipSuccess) return hip_fail(e, "map copy");
    }
    if ((e = hipEventRecord(p_->ev_copied[buf], p_->side)) != hipSuccess) return hip_fail(e, "event record");
    if ((e = hipStreamWaitEvent(hs_, p_->ev_copied[buf], 0)) != hipSuccess) return hip_fail(e, "stream wait");
    for (int i = 0; i < g; ++i) {
      char* src = mb + i * p_->layer_bytes;
      if (q8_) {
        dp_.q[i] = reinterpret_cast<const int8_t*>(src);
        dp_.s[i] = reinterpret_cast<const uint16_t*>(src + p_->scale_off);
        dp_.w[i] = dq_ + i * elems;
      }
      mp.a[i] = q8_ ? dq_ + i * elems : reinterpret_cast<const uint16_t*>(src);
      mp.b[i] = reinterpret_cast<const uint16_t*>(src + p_->bias_off);
    }
    if (q8_) {
      Timed tm(p_, RF_K_DEQUANT, hs_);
      if ((e = rf::launch_dequant(dp_, g, hs_)) != hipSuccess) return hip_fail(e, "dequant launch");
    }
    last_buf_ = buf;
    ++calls_;
    return RF_OK;
  }

  // Call after the last kernel that reads the group just loaded is enqueued.
  rf_status consumed() {
    if (!host_) return RF_OK;
    hipError_t e = hipEventRecord(p_->ev_consumed[last_buf_], hs_);
    return e == hipSuccess ? RF_OK : hip_fail(e, "event record");
  }

 private:
  rf_plan* p_;
  const MapSrc& maps_;
  uint16_t* dq_;
  hipStream_t hs_;
  bool q8_, host_;
  int calls_ = 0, last_buf_ = 0;  // streamed groups loaded so far; buffer of the last
  rf::DequantParams dp_{};
};

// Largest layer group (<= max_group) whose workspace fits.
template <class F>
int pick_group(const rf_plan* p, size_t ws_bytes, F bytes_for) {
  for (int g = max_group(p); g > 1; --g)
    if (bytes_for(g) <= ws_bytes) return g;
  return 1;
}

rf_status check_opts(const rf_plan* p, const rf_fill_opts* o) {
  const int L = p->s.n_late;
  rf_status st;
  if (o && o->k_norm)
    if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(o->k_norm), L, "k_norm")) != RF_OK) return st;
  const bool has_idx = o && (o->w_idx || o->idx_cache);
  if (p->s.n_idx == 0)
    return has_idx ? fail(RF_E_ARG, "w_idx / idx_cache given but the plan has n_idx = 0") : RF_OK;
  if (!o || !o->w_idx || !o->idx_cache)
    return fail(RF_E_ARG, "the plan has n_idx=%d indexer heads: opts->w_idx and opts->idx_cache are required",
                p->s.n_idx);
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(o->w_idx), L, "w_idx")) != RF_OK) return st;
  return check_layer_ptrs(reinterpret_cast<const void* const*>(o->idx_cache), L, "idx_cache");
}

rf_status check_vscale(const rf_plan* p, const rf_vscale* vs) {
  if (!vs) return RF_OK;
  if (!vs->scale || !vs->group_of_row) return fail(RF_E_ARG, "vscale has a null scale or group_of_row");
  if (vs->n_groups < 1) return fail(RF_E_ARG, "vscale n_groups=%d must be >= 1", vs->n_groups);
  if (reinterpret_cast<uintptr_t>(vs->scale) & 3) return fail(RF_E_ARG, "vscale scale is not 4-byte aligned");
  return RF_OK;
}

// Workspace of the value-scale measurement, in carve order.
struct ScaleWs {
  size_t prep, y, dq, v, ratio, pos, ssq, rs, total;
};
ScaleWs scale_ws(const rf_plan* p, int n, int g) {
  const rf_shape& s = p->s;
  ScaleWs r{};
  r.prep = prep_bytes(s, g);
  r.y = y_bytes(s, n, g);
  r.dq = dq_bytes(s, p->flags, g);
  r.v = up(static_cast<size_t>(g) * n * kv_width(s) * 2);
  r.ratio = up(static_cast<size_t>(s.n_late) * n * s.n_kv * 4);
  r.pos = up(static_cast<size_t>(std::max(n, 1)) * 4);
  r.ssq = ssq_bytes(s, n, g);
  r.rs = rs_bytes(n, g);
  r.total = kFlagBytes + r.prep + r.y + r.dq + 2 * r.v + r.ratio + r.pos + r.ssq + r.rs;
  return r;
}

// The value-scale measurement of one layer group, on a workspace carved as
// ScaleWs (its prep and dq parts unused here): predicted values of the
// calibration rows from the group's maps, exact values from the true inputs,
// their per-head norm ratios, and the per-request means for the group's layers.
class ScaleMeasure {
 public:
  ScaleMeasure(rf_plan* p, hipStream_t hs, void* ws, int G, const uint16_t* x, int64_t ld_x,
               const uint16_t* const* layer_in, int64_t ld_in, const int32_t* calib_rows, const int32_t* calib_group,
               int n, int n_groups, const uint16_t* prep, int wrows)
      : p_(p), hs_(hs), s_(p->s), layer_in_(layer_in), ld_in_(ld_in), calib_group_(calib_group), n_(n),
        n_groups_(n_groups) {
    const ScaleWs sw = scale_ws(p, n, G);
    char* c = static_cast<char*>(ws) + kFlagBytes + sw.prep;
    ybuf_ = reinterpret_cast<uint16_t*>(c);
    ve_ = reinterpret_cast<uint16_t*>(c += sw.y + sw.dq);
    vp_ = reinterpret_cast<uint16_t*>(c += sw.v);
    ratio_ = reinterpret_cast<float*>(c += sw.v);
    zero_pos_ = reinterpret_cast<int32_t*>(c += sw.ratio);
    ssq_ = reinterpret_cast<float*>(c += sw.pos);
    rsb_ = reinterpret_cast<float*>(c += sw.ssq);
    const int w = kv_width(s_);
    mp_.x = x;
    mp_.ld_x = ld_x;
    mp_.rows = calib_rows;
    mp_.n_rows = s_.n_rows;
    mp_.M = n;
    mp_.K = s_.d_in;
    mp_.N = s_.d_out;
    mp_.tiles_m = (n + rf::kTileM - 1) / rf::kTileM;
    mp_.tiles_n = s_.d_out / rf::kTileN;
    mp_.y = ybuf_;
    mp_.ssq = ssq_;
    // Value features only, row m of the call stored densely at row m (slot =
    // row, rows numbered 0..n-1; positions are not used by values).
    kp_.n_in_rows = n;
    kp_.M = n;
    kp_.K = s_.d_out;
    kp_.w = w;
    kp_.head_dim = s_.head_dim;
    kp_.tiles_m = mp_.tiles_m;
    kp_.tiles_n = (2 * w - w / rf::kTileN * rf::kTileN) / rf::kTileN;
    kp_.wrows = wrows;
    kp_.wkv = prep;
    kp_.positions = zero_pos_;
    kp_.n_rows = n;
    kp_.n_slots = n;
    kp_.max_pos = s_.max_pos;
    kp_.eps = s_.rms_eps;
    kp_.n_kv = s_.n_kv;
    kp_.v_only = 1;
    rp_.n = n;
    rp_.n_kv = s_.n_kv;
    rp_.head_dim = s_.head_dim;
    rmp_.ld_in = ld_in;
    rmp_.n_in_rows = n;
    rmp_.M = n;
    rmp_.K = s_.d_out;
    rmp_.inv_k = 1.0f / s_.d_out;
    rmp_.eps = s_.rms_eps;
    rmp_.rs = rsb_;
  }

  rf_status begin() {
    if (n_ == 0) return RF_OK;
    hipError_t e = rf::launch_zero_i32(zero_pos_, n_, hs_);
    return e == hipSuccess ? RF_OK : hip_fail(e, "clear launch");
  }

  // The calibration rows through the maps of layers l0 .. l0+g-1 (device
  // maps in maps.a / maps.b); then finish().
  rf_status group(int l0, int g, const rf::MapParams& maps) {
    hipError_t e;
    const size_t v_layer = static_cast<size_t>(n_) * kv_width(s_);
    if (n_ > 0) {
      for (int i = 0; i < g; ++i) {
        mp_.a[i] = maps.a[i];
        mp_.b[i] = maps.b[i];
        rp_.ve[i] = ve_ + i * v_layer;
        rp_.vp[i] = vp_ + i * v_layer;
        rp_.ratio[i] = ratio_ + static_cast<size_t>(l0 + i) * n_ * s_.n_kv;
      }
      Timed tm(p_, RF_K_SCALE, hs_);
      if ((e = rf::launch_map(mp_, g, hs_)) != hipSuccess) return hip_fail(e, "map launch");
    }
    return RF_OK;
  }

  // The rest of the group once the maps may be released: predicted values
  // from the map's output (norms from its row sums), exact values from the
  // true inputs (norms from a pass over them), ratios, and the means of the
  // group's layers into scale [n_late][n_groups][n_kv].
  rf_status finish(int l0, int g, float* scale) {
    hipError_t e;
    const int w = kv_width(s_);
    const size_t y_layer = static_cast<size_t>(n_) * s_.d_out;
    const size_t v_layer = static_cast<size_t>(n_) * w;
    if (n_ > 0) {
      {
        Timed tm(p_, RF_K_SCALE, hs_);
        if ((e = rf::launch_row_scale(ssq_, mp_.tiles_n, n_, g, 1.0f / s_.d_out, s_.rms_eps, rsb_, hs_)) != hipSuccess)
          return hip_fail(e, "row scale launch");
      }
      kp_.ld_in = s_.d_out;
      for (int i = 0; i < g; ++i) {
        kp_.in[i] = ybuf_ + i * y_layer;
        kp_.vc[i] = vp_ + i * v_layer;
        kp_.rs[i] = rsb_ + static_cast<size_t>(i) * n_;
      }
      {
        Timed tm(p_, RF_K_SCALE, hs_);
        if ((e = rf::launch_kv(kp_, g, hs_)) != hipSuccess) return hip_fail(e, "kv launch");
      }
      kp_.ld_in = ld_in_;
      for (int i = 0; i < g; ++i) {
        kp_.in[i] = layer_in_[l0 + i];
        kp_.vc[i] = ve_ + i * v_layer;
        rmp_.in[i] = layer_in_[l0 + i];
      }
      {
        // (the same stream: the predicted launch above has read rsb)
        Timed tm(p_, RF_K_SCALE, hs_);
        if ((e = rf::launch_row_rms(rmp_, g, hs_)) != hipSuccess) return hip_fail(e, "row rms launch");
      }
      {
        Timed tm(p_, RF_K_SCALE, hs_);
        if ((e = rf::launch_kv(kp_, g, hs_)) != hipSuccess) return hip_fail(e, "kv launch");
      }
      {
        Timed tm(p_, RF_K_SCALE, hs_);
        if ((e = rf::launch_head_ratio(rp_, g, hs_)) != hipSuccess) return hip_fail(e, "ratio launch");
      }
    }
    Timed tm(p_, RF_K_SCALE, hs_);
    const size_t per_layer_ratio = static_cast<size_t>(n_) * s_.n_kv;
    const size_t per_layer_scale = static_cast<size_t>(n_groups_) * s_.n_kv;
    if ((e = rf::launch_scale_mean(ratio_ + l0 * per_layer_ratio, calib_group_, n_, s_.n_kv, n_groups_, g,
                                   scale + l0 * per_layer_scale, hs_)) != hipSuccess)
      return hip_fail(e, "scale launch");
    return RF_OK;
  }

 private:
  rf_plan* p_;
  hipStream_t hs_;
  const rf_shape& s_;
  const uint16_t* const* layer_in_;
  int64_t ld_in_;
  const int32_t* calib_group_;
  int n_, n_groups_;
  uint16_t *ybuf_, *ve_, *vp_;
  float *ratio_, *ssq_, *rsb_;
  int32_t* zero_pos_;
  rf::MapParams mp_{};
  rf::KvParams kp_{};
  rf::RatioParams rp_{};
  rf::RmsParams rmp_{};
};

rf_status check_measure_args(const rf_plan* p, const uint16_t* const* layer_in, int64_t ld_in,
                             const int32_t* calib_rows, const int32_t* calib_group, int32_t n, int32_t n_groups) {
  const rf_shape& s = p->s;
  if (n < 0 || n > s.n_rows) return fail(RF_E_ARG, "n_calib=%d outside [0, n_rows=%d]", n, s.n_rows);
  if (n_groups < 1) return fail(RF_E_ARG, "n_groups=%d must be >= 1", n_groups);
  if (ld_in < s.d_out || ld_in % 8)
    return fail(RF_E_ARG, "ld_in=%lld must be >= d_out and a multiple of 8", (long long)ld_in);
  if (n > 0 && (!calib_rows || !calib_group)) return fail(RF_E_ARG, "calib_rows or calib_group is null");
  return check_layer_ptrs(reinterpret_cast<const void* const*>(layer_in), s.n_late, "layer_in");
}

rf_status fill_impl(rf_plan* p, const char* fn, const uint16_t* x, int64_t ld_x, const int32_t* fill_rows,
                    int32_t n_fill, const int32_t* positions, const int32_t* slot_of_row, const MapSrc& maps,
                    const uint16_t* const* gamma, const uint16_t* const* w_k, const uint16_t* const* w_v,
                    const float* rope, uint16_t* const* k_cache, uint16_t* const* v_cache, const rf_fill_opts* opts,
                    void* ws, size_t ws_bytes, void* stream) {
  const rf_shape& s = p->s;
  const rf_vmeasure* meas_in = opts ? opts->measure : nullptr;
  // with a measurement, its scales are applied like an rf_vscale
  const rf_vscale measured{meas_in ? meas_in->scale : nullptr, meas_in ? meas_in->group_of_row : nullptr,
                           meas_in ? meas_in->n_groups : 0};
  const rf_vscale* vscale = meas_in ? &measured : (opts ? opts->vscale : nullptr);
  const uint16_t* const* k_norm = opts ? opts->k_norm : nullptr;
  const int L = s.n_late;
  rf_status st;
  if ((st = check_maps(p, fn, maps)) != RF_OK) return st;
  if (meas_in) {
    if (opts->vscale) return fail(RF_E_ARG, "give opts->vscale or opts->measure, not both");
    if ((st = check_measure_args(p, meas_in->layer_in, meas_in->ld_in, meas_in->calib_rows, meas_in->calib_group,
                                 meas_in->n_calib, meas_in->n_groups)) != RF_OK)
      return st;
    const size_t m1 = rf_value_scales_workspace_bytes(p, meas_in->n_calib, 1);
    if (!meas_in->workspace || (reinterpret_cast<uintptr_t>(meas_in->workspace) % kAlign) || meas_in->ws_bytes < m1)
      return fail(RF_E_WORKSPACE, "measure workspace of %zu bytes given, %zu needed (256-byte aligned)",
                  meas_in->ws_bytes, m1);
  }
  if (n_fill < 0 || n_fill > s.n_rows) return fail(RF_E_ARG, "n_fill=%d outside [0, n_rows=%d]", n_fill, s.n_rows);
  if (!x || !aligned16(x)) return fail(RF_E_ARG, "x is null or not 16-byte aligned");
  if (ld_x < s.d_in || ld_x % 8) return fail(RF_E_ARG, "ld_x=%lld must be >= d_in and a multiple of 8", (long long)ld_x);
  if (n_fill > 0 && !fill_rows) return fail(RF_E_ARG, "fill_rows is null");
  if (!positions) return fail(RF_E_ARG, "positions is null");
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(gamma), L, "gamma")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(w_k), L, "w_k")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(w_v), L, "w_v")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(k_cache), L, "k_cache")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(v_cache), L, "v_cache")) != RF_OK) return st;
  if ((st = check_vscale(p, vscale)) != RF_OK) return st;
  if ((st = check_opts(p, opts)) != RF_OK) return st;
  if (rope && !aligned16(rope)) return fail(RF_E_ARG, "rope table is not 16-byte aligned");
  const size_t need1 = rf_fill_workspace_bytes(p, n_fill, 1);
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign) || ws_bytes < need1)
    return fail(RF_E_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)", ws_bytes, need1);
  if (n_fill == 0) return RF_OK;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  int G = pick_group(p, ws_bytes, [&](int g) { return rf_fill_workspace_bytes(p, n_fill, g); });
  if (meas_in)
    G = std::min(G, pick_group(p, meas_in->ws_bytes,
                               [&](int g) { return rf_value_scales_workspace_bytes(p, meas_in->n_calib, g); }));

  char* w0 = static_cast<char*>(ws);
  float* rope_ws = reinterpret_cast<float*>(w0);
  int32_t* flag = reinterpret_cast<int32_t*>(w0 + rope_bytes(s));
  uint16_t* prep = reinterpret_cast<uint16_t*>(w0 + rope_bytes(s) + kFlagBytes);
  uint16_t* ybuf = reinterpret_cast<uint16_t*>(w0 + rope_bytes(s) + kFlagBytes + prep_bytes(s, G));
  uint16_t* dq = reinterpret_cast<uint16_t*>(w0 + rope_bytes(s) + kFlagBytes + prep_bytes(s, G) +
                                             y_bytes(s, n_fill, G));
  float* ssq = reinterpret_cast<float*>(reinterpret_cast<char*>(dq) + dq_bytes(s, p->flags, G));
  float* rsb = reinterpret_cast<float*>(reinterpret_cast<char*>(ssq) + ssq_bytes(s, n_fill, G));

  hipError_t e;
  if (p->flags & RF_VALIDATE)
    if ((st = run_validate(p, fill_rows, n_fill, 1, positions, slot_of_row, flag, hs)) != RF_OK) return st;
  if (!rope) {
    Timed tm(p, RF_K_ROPE, hs);
    if ((e = rf::launch_rope_table(rope_ws, s.max_pos, s.head_dim, s.rope_theta, hs)) != hipSuccess)
      return hip_fail(e, "rope table launch");
    rope = rope_ws;
  }

  const int w = kv_width(s);
  rf::MapParams mp{};
  mp.x = x;
  mp.ld_x = ld_x;
  mp.rows = fill_rows;
  mp.n_rows = s.n_rows;
  mp.M = n_fill;
  mp.K = s.d_in;
  mp.N = s.d_out;
  mp.tiles_m = (n_fill + rf::kTileM - 1) / rf::kTileM;
  mp.tiles_n = s.d_out / rf::kTileN;
  mp.y = ybuf;
  mp.ssq = ssq;

  rf::KvParams kp{};
  kp.ld_in = s.d_out;
  kp.in_rows = nullptr;
  kp.n_in_rows = n_fill;
  kp.out_rows = fill_rows;
  kp.M = n_fill;
  kp.K = s.d_out;
  kp.w = w;
  kp.head_dim = s.head_dim;
  kp.tiles_m = mp.tiles_m;
  kp.tall_f0 = tall_f0(s, n_fill, s.d_out);
  kp.tiles_n = (kp.tall_f0 >= 0 ? kp.tall_f0 : prep_rows(s)) / rf::kTileN;
  kp.wrows = prep_rows(s);
  kp.widx = idx_width(s);
  kp.wkv = prep;
  kp.positions = positions;
  kp.slots = slot_of_row;
  kp.n_rows = s.n_rows;
  kp.n_slots = s.n_slots;
  kp.max_pos = s.max_pos;
  kp.rope = rope;
  kp.eps = s.rms_eps;
  kp.n_kv = s.n_kv;
  kp.n_groups = vscale ? vscale->n_groups : 0;
  kp.group_of_row = vscale ? vscale->group_of_row : nullptr;
  kp.qk_norm = k_norm != nullptr;

  rf::PrepParams pp{};
  pp.d = s.d_out;
  pp.w = w;
  pp.widx = idx_width(s);
  pp.rows = prep_rows(s);
  pp.out = prep;

  const size_t y_layer = static_cast<size_t>(n_fill) * s.d_out;
  const size_t vs_layer = vscale ? static_cast<size_t>(vscale->n_groups) * s.n_kv : 0;
  MapFeeder feed(p, maps, dq, hs);
  if ((st = feed.begin()) != RF_OK) return st;
  // The in-fill measurement runs on the plan's measurement stream, beside
  // the fill's own launches: each group's measurement starts once the
  // group's prepared weights and maps are in place on the fill's stream, and
  // the group's K/V launch waits for its scales.  Its kernels and inputs are
  // those of rf_value_scales, so the scales are the same bytes; only the
  // small launches now overlap the group's map contraction instead of
  // queueing behind it.  Every exit joins the two streams again.
  std::unique_ptr<ScaleMeasure> meas;
  struct Join {
    rf_plan* p = nullptr;
    hipStream_t hs = nullptr;
    ~Join() {
      if (p && hipEventRecord(p->from_meas, p->meas) == hipSuccess) (void)hipStreamWaitEvent(hs, p->from_meas, 0);
    }
  } join;
  auto to_meas = [&]() -> rf_status {
    hipError_t er = hipEventRecord(p->to_meas, hs);
    if (er == hipSuccess) er = hipStreamWaitEvent(p->meas, p->to_meas, 0);
    return er == hipSuccess ? RF_OK : hip_fail(er, "measurement stream wait");
  };
  if (meas_in) {
    if ((e = p->make_meas_stream()) != hipSuccess) return hip_fail(e, "measurement stream");
    if ((st = to_meas()) != RF_OK) return st;
    join.p = p;
    join.hs = hs;
    meas.reset(new ScaleMeasure(p, p->meas, meas_in->workspace, G, x, ld_x, meas_in->layer_in, meas_in->ld_in,
                                meas_in->calib_rows, meas_in->calib_group, meas_in->n_calib, meas_in->n_groups, prep,
                                prep_rows(s)));
    if ((st = meas->begin()) != RF_OK) return st;
  }
  for (int l0 = 0, g = 0; l0 < L; l0 += g) {
    g = group_at(p, l0, G);
    for (int i = 0; i < g; ++i) {
      pp.gamma[i] = gamma[l0 + i];
      pp.wk[i] = w_k[l0 + i];
      pp.wv[i] = w_v[l0 + i];
      pp.wi[i] = s.n_idx ? opts->w_idx[l0 + i] : nullptr;
      kp.in[i] = ybuf + i * y_layer;
      kp.rs[i] = rsb + static_cast<size_t>(i) * n_fill;
      kp.kc[i] = k_cache[l0 + i];
      kp.ic[i] = s.n_idx ? opts->idx_cache[l0 + i] : nullptr;
      kp.vc[i] = v_cache[l0 + i];
      kp.vscale[i] = vscale ? vscale->scale + (l0 + i) * vs_layer : nullptr;
      kp.kgamma[i] = k_norm ? k_norm[l0 + i] : nullptr;
    }
    {
      Timed tm(p, RF_K_PREP, hs);
      if ((e = rf::launch_prep(pp, g, hs)) != hipSuccess) return hip_fail(e, "prep launch");
    }
    if ((st = feed.load(l0, g, mp)) != RF_OK) return st;
    // the measurement's calibration rows go through the same loaded maps
    // (and prepared weights), on the measurement stream
    if (meas && (st = to_meas()) != RF_OK) return st;
    {
      Timed tm(p, RF_K_MAP, hs);
      if ((e = rf::launch_map(mp, g, hs)) != hipSuccess) return hip_fail(e, "map launch");
    }
    if (meas) {
      if ((st = meas->group(l0, g, mp)) != RF_OK) return st;
      if ((st = meas->finish(l0, g, meas_in->scale)) != RF_OK) return st;
      if ((e = hipEventRecord(p->from_meas, p->meas)) != hipSuccess) return hip_fail(e, "event record");
    }
    {
      Timed tm(p, RF_K_NORM, hs);
      if ((e = rf::launch_row_scale(ssq, mp.tiles_n, n_fill, g, 1.0f / s.d_out, s.rms_eps, rsb, hs)) != hipSuccess)
        return hip_fail(e, "row scale launch");
    }
    // the group's scales are in place before its K/V launch, and the
    // measurement has read the group's maps before their buffer is released
    if (meas && (e = hipStreamWaitEvent(hs, p->from_meas, 0)) != hipSuccess) return hip_fail(e, "stream wait");
    if ((st = feed.consumed()) != RF_OK) return st;
    {
      Timed tm(p, RF_K_KV, hs);
      if ((e = rf::launch_kv(kp, g, hs)) != hipSuccess) return hip_fail(e, "kv launch");
    }
  }
  return RF_OK;
}

rf_status value_scales_impl(rf_plan* p, const char* fn, const uint16_t* x, int64_t ld_x,
                            const uint16_t* const* layer_in, int64_t ld_in, const int32_t* calib_rows,
                            const int32_t* calib_group, int32_t n, int32_t n_groups, const MapSrc& maps,
                            const uint16_t* const* gamma, const uint16_t* const* w_v, float* scale, void* ws,
                            size_t ws_bytes, void* stream) {
  const rf_shape& s = p->s;
  const int L = s.n_late;
  rf_status st;
  if ((st = check_maps(p, fn, maps)) != RF_OK) return st;
  if ((st = check_measure_args(p, layer_in, ld_in, calib_rows, calib_group, n, n_groups)) != RF_OK) return st;
  if (!x || !aligned16(x)) return fail(RF_E_ARG, "x is null or not 16-byte aligned");
  if (ld_x < s.d_in || ld_x % 8) return fail(RF_E_ARG, "ld_x=%lld must be >= d_in and a multiple of 8", (long long)ld_x);
  if (!scale || (reinterpret_cast<uintptr_t>(scale) & 3)) return fail(RF_E_ARG, "scale is null or misaligned");
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(gamma), L, "gamma")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(w_v), L, "w_v")) != RF_OK) return st;
  const size_t need1 = rf_value_scales_workspace_bytes(p, n, 1);
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign) || ws_bytes < need1)
    return fail(RF_E_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)", ws_bytes, need1);

  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int G = pick_group(p, ws_bytes, [&](int g) { return rf_value_scales_workspace_bytes(p, n, g); });
  const ScaleWs sw = scale_ws(p, n, G);
  char* c = static_cast<char*>(ws) + kFlagBytes;
  uint16_t* prep = reinterpret_cast<uint16_t*>(c);
  uint16_t* dq = reinterpret_cast<uint16_t*>(c + sw.prep + sw.y);
  const int w = kv_width(s);
  ScaleMeasure meas(p, hs, ws, G, x, ld_x, layer_in, ld_in, calib_rows, calib_group, n, n_groups, prep, 2 * w);
  if ((st = meas.begin()) != RF_OK) return st;
  rf::PrepParams pp{};
  pp.d = s.d_out;
  pp.w = w;
  pp.rows = 2 * w;  // keys and values only (no indexer rows here)
  pp.out = prep;
  MapFeeder feed(p, maps, dq, hs);
  if (n > 0 && (st = feed.begin()) != RF_OK) return st;
  hipError_t e;
  for (int l0 = 0, g = 0; l0 < L; l0 += g) {
    g = group_at(p, l0, G);
    if (n > 0) {
      for (int i = 0; i < g; ++i) {
        pp.gamma[i] = gamma[l0 + i];
        pp.wk[i] = w_v[l0 + i];  // the key half of the prepared weights is not used
        pp.wv[i] = w_v[l0 + i];
      }
      {
        Timed tm(p, RF_K_SCALE, hs);
        if ((e = rf::launch_prep(pp, g, hs)) != hipSuccess) return hip_fail(e, "prep launch");
      }
      rf::MapParams mp{};
      if ((st = feed.load(l0, g, mp)) != RF_OK) return st;
      if ((st = meas.group(l0, g, mp)) != RF_OK) return st;
      if ((st = feed.consumed()) != RF_OK) return st;
    }
    if ((st = meas.finish(l0, g, scale)) != RF_OK) return st;
  }
  return RF_OK;
}

}  // namespace

extern "C" {

rf_status rf_fill(rf_plan* p, const uint16_t* x, int64_t ld_x, const int32_t* fill_rows, int32_t n_fill,
                  const int32_t* positions, const int32_t* slot_of_row, const uint16_t* const* map_a,
                  const uint16_t* const* map_b, const uint16_t* const* gamma, const uint16_t* const* w_k,
                  const uint16_t* const* w_v, const float* rope, uint16_t* const* k_cache,
                  uint16_t* const* v_cache, const rf_fill_opts* opts, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return fail(RF_E_ARG, "plan is null");
  MapSrc m;
  m.a = map_a;
  m.b = map_b;
  return fill_impl(p, "rf_fill", x, ld_x, fill_rows, n_fill, positions, slot_of_row, m, gamma, w_k, w_v, rope,
                   k_cache, v_cache, opts, ws, ws_bytes, stream);
}

rf_status rf_fill_q8(rf_plan* p, const uint16_t* x, int64_t ld_x, const int32_t* fill_rows, int32_t n_fill,
                     const int32_t* positions, const int32_t* slot_of_row, const int8_t* const* map_q,
                     const uint16_t* const* map_scale, const uint16_t* const* map_b, const uint16_t* const* gamma,
                     const uint16_t* const* w_k, const uint16_t* const* w_v, const float* rope,
                     uint16_t* const* k_cache, uint16_t* const* v_cache, const rf_fill_opts* opts, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!p) return fail(RF_E_ARG, "plan is null");
  if (!map_q || !map_scale) return fail(RF_E_ARG, "map_q or map_scale array is null");
  MapSrc m;
  m.q = map_q;
  m.scale = map_scale;
  m.b = map_b;
  return fill_impl(p, "rf_fill_q8", x, ld_x, fill_rows, n_fill, positions, slot_of_row, m, gamma, w_k, w_v, rope,
                   k_cache, v_cache, opts, ws, ws_bytes, stream);
}

size_t rf_value_scales_workspace_bytes(const rf_plan* p, int32_t n_calib, int32_t g) {
  if (!p || n_calib < 0 || g < 1 || g > p->s.n_late) return 0;
  g = std::min(g, max_group(p));
  return scale_ws(p, n_calib, g).total;
}

rf_status rf_value_scales(rf_plan* p, const uint16_t* x, int64_t ld_x, const uint16_t* const* layer_in,
                          int64_t ld_in, const int32_t* calib_rows, const int32_t* calib_group, int32_t n_calib,
                          int32_t n_groups, const uint16_t* const* map_a, const uint16_t* const* map_b,
                          const uint16_t* const* gamma, const uint16_t* const* w_v, float* scale, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!p) return fail(RF_E_ARG, "plan is null");
  MapSrc m;
  m.a = map_a;
  m.b = map_b;
  return value_scales_impl(p, "rf_value_scales", x, ld_x, layer_in, ld_in, calib_rows, calib_group, n_calib,
                           n_groups, m, gamma, w_v, scale, ws, ws_bytes, stream);
}

rf_status rf_value_scales_q8(rf_plan* p, const uint16_t* x, int64_t ld_x, const uint16_t* const* layer_in,
                             int64_t ld_in, const int32_t* calib_rows, const int32_t* calib_group, int32_t n_calib,
                             int32_t n_groups, const int8_t* const* map_q, const uint16_t* const* map_scale,
                             const uint16_t* const* map_b, const uint16_t* const* gamma,
                             const uint16_t* const* w_v, float* scale, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return fail(RF_E_ARG, "plan is null");
  if (!map_q || !map_scale) return fail(RF_E_ARG, "map_q or map_scale array is null");
  MapSrc m;
  m.q = map_q;
  m.scale = map_scale;
  m.b = map_b;
  return value_scales_impl(p, "rf_value_scales_q8", x, ld_x, layer_in, ld_in, calib_rows, calib_group, n_calib,
                           n_groups, m, gamma, w_v, scale, ws, ws_bytes, stream);
}

rf_status rf_map_dequantize_q8(const int8_t* q, const uint16_t* scale, int32_t d_out, int32_t d_in, uint16_t* w,
                               void* stream) {
  if (!q || !scale || !w) return fail(RF_E_ARG, "null argument");
  if (!aligned16(q) || !aligned16(w)) return fail(RF_E_ARG, "q and w must be 16-byte aligned");
  if (d_out < 1 || d_in < 1 || d_in % rf::kQ8Block)
    return fail(RF_E_SHAPE, "d_out must be >= 1 and d_in a positive multiple of %d", rf::kQ8Block);
  rf::DequantParams dp{};
  dp.d_out = d_out;
  dp.d_in = d_in;
  dp.q[0] = q;
  dp.s[0] = scale;
  dp.w[0] = w;
  hipError_t e = rf::launch_dequant(dp, 1, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RF_OK : hip_fail(e, "dequant launch");
}

rf_status rf_kv_project(rf_plan* p, const uint16_t* const* layer_in, int64_t ld_in, const int32_t* rows, int32_t n,
                        const int32_t* positions, const int32_t* slot_of_row, const uint16_t* const* gamma,
                        const uint16_t* const* w_k, const uint16_t* const* w_v, const float* rope,
                        uint16_t* const* k_cache, uint16_t* const* v_cache, const rf_fill_opts* opts, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!p) return fail(RF_E_ARG, "plan is null");
  if (opts && opts->vscale) return fail(RF_E_ARG, "rf_kv_project writes exact rows: no value rescale");
  const rf_shape& s = p->s;
  const int L = s.n_late;
  if (n < 0 || n > s.n_rows) return fail(RF_E_ARG, "n=%d outside [0, n_rows=%d]", n, s.n_rows);
  if (ld_in < s.d_out || ld_in % 8) return fail(RF_E_ARG, "ld_in=%lld must be >= d_out and a multiple of 8", (long long)ld_in);
  if (n > 0 && !rows) return fail(RF_E_ARG, "rows is null");
  if (!positions) return fail(RF_E_ARG, "positions is null");
  rf_status st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(layer_in), L, "layer_in")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(gamma), L, "gamma")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(w_k), L, "w_k")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(w_v), L, "w_v")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(k_cache), L, "k_cache")) != RF_OK) return st;
  if ((st = check_layer_ptrs(reinterpret_cast<const void* const*>(v_cache), L, "v_cache")) != RF_OK) return st;
  if ((st = check_opts(p, opts)) != RF_OK) return st;
  if (rope && !aligned16(rope)) return fail(RF_E_ARG, "rope table is not 16-byte aligned");
  const size_t need1 = rf_kv_project_workspace_bytes(p, 1);
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign) || ws_bytes < need1)
    return fail(RF_E_WORKSPACE, "workspace of %zu bytes given, %zu needed (256-byte aligned)", ws_bytes, need1);
  if (n == 0) return RF_OK;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  int G = 1;
  for (int g = std::min(s.n_late, rf::kMaxGroup); g > 1; --g)  // no maps here: any plan groups freely
    if (rf_kv_project_workspace_bytes(p, g) <= ws_bytes) {
      G = g;
      break;
    }
  char* w0 = static_cast<char*>(ws);
  float* rope_ws = reinterpret_cast<float*>(w0);
  int32_t* flag = reinterpret_cast<int32_t*>(w0 + rope_bytes(s));
  uint16_t* prep = reinterpret_cast<uint16_t*>(w0 + rope_bytes(s) + kFlagBytes);
  float* rsb = reinterpret_cast<float*>(w0 + rope_bytes(s) + kFlagBytes + prep_bytes(s, G));
  hipError_t e;
  if (p->flags & RF_VALIDATE)
    if ((st = run_validate(p, rows, n, 0, positions, slot_of_row, flag, hs)) != RF_OK) return st;
  if (!rope) {
    Timed tm(p, RF_K_ROPE, hs);
    if ((e = rf::launch_rope_table(rope_ws, s.max_pos, s.head_dim, s.rope_theta, hs)) != hipSuccess)
      return hip_fail(e, "rope table launch");
    rope = rope_ws;
  }
  const int w = kv_width(s);
  rf::KvParams kp{};
  kp.ld_in = ld_in;
  kp.in_rows = rows;
  kp.n_in_rows = s.n_rows;
  kp.out_rows = rows;
  kp.M = n;
  kp.K = s.d_out;
  kp.w = w;
  kp.head_dim = s.head_dim;
  kp.tiles_m = (n + rf::kTileM - 1) / rf::kTileM;
  kp.tall_f0 = tall_f0(s, s.n_rows, ld_in);
  kp.tiles_n = (kp.tall_f0 >= 0 ? kp.tall_f0 : prep_rows(s)) / rf::kTileN;
  kp.wrows = prep_rows(s);
  kp.widx = idx_width(s);
  kp.wkv = prep;
  kp.positions = positions;
  kp.slots = slot_of_row;
  kp.n_rows = s.n_rows;
  kp.n_slots = s.n_slots;
  kp.max_pos = s.max_pos;
  kp.rope = rope;
  kp.eps = s.rms_eps;
  kp.n_kv = s.n_kv;
  const uint16_t* const* k_norm = opts ? opts->k_norm : nullptr;
  kp.qk_norm = k_norm != nullptr;
  rf::PrepParams pp{};
  pp.d = s.d_out;
  pp.w = w;
  pp.widx = idx_width(s);
  pp.rows = prep_rows(s);
  pp.out = prep;
  rf::RmsParams rp{};
  rp.ld_in = ld_in;
  rp.in_rows = rows;
  rp.n_in_rows = s.n_rows;
  rp.M = n;
  rp.K = s.d_out;
  rp.inv_k = 1.0f / s.d_out;
  rp.eps = s.rms_eps;
  rp.rs = rsb;
  for (int l0 = 0, g = 0; l0 < L; l0 += g) {
    g = group_at(p, l0, G);
    for (int i = 0; i < g; ++i) {
      pp.gamma[i] = gamma[l0 + i];
      pp.wk[i] = w_k[l0 + i];
      pp.wv[i] = w_v[l0 + i];
      pp.wi[i] = s.n_idx ? opts->w_idx[l0 + i] : nullptr;
      kp.in[i] = layer_in[l0 + i];
      rp.in[i] = layer_in[l0 + i];
      kp.rs[i] = rsb + static_cast<size_t>(i) * n;
      kp.kc[i] = k_cache[l0 + i];
      kp.ic[i] = s.n_idx ? opts->idx_cache[l0 + i] : nullptr;
      kp.vc[i] = v_cache[l0 + i];
      kp.kgamma[i] = k_norm ? k_norm[l0 + i] : nullptr;
    }
    {
      Timed tm(p, RF_K_PREP, hs);
      if ((e = rf::launch_prep(pp, g, hs)) != hipSuccess) return hip_fail(e, "prep launch");
    }
    {
      Timed tm(p, RF_K_NORM, hs);
      if ((e = rf::launch_row_rms(rp, g, hs)) != hipSuccess) return hip_fail(e, "row rms launch");
    }
    {
      Timed tm(p, RF_K_KV, hs);
      if ((e = rf::launch_kv(kp, g, hs)) != hipSuccess) return hip_fail(e, "kv launch");
    }
  }
  return RF_OK;
}

}  // extern "C"
