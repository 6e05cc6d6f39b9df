// C ABI of libsrp (include/srp.h): argument checks, rotary tables, workspace
// carve-up and the launch sequence of one fused layer on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "kernels.hpp"

using namespace srp;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define SRP_HIP(call)                                                             \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess)                                                         \
      return fail(SRP_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_));      \
  } while (0)

// ------------------------------------------------------------------------- //
// rotary tables: one per (device, head_dim, base), grown on demand. cos/sin of
// p * base^(-2i/d) are evaluated in double on the host and rounded to float.
// Superseded tables stay allocated so in-flight work never reads freed memory.
// ------------------------------------------------------------------------- //
struct Table {
  float *cos_t = nullptr, *sin_t = nullptr;
  int max_pos = 0;
};
std::mutex g_mu;
std::map<std::tuple<int, int, double>, Table> g_tables;
std::vector<void *> g_retired;

int get_table(int d, double base, int max_pos, RopeTable *out) {
  int dev = 0;
  SRP_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_mu);
  Table &t = g_tables[std::make_tuple(dev, d, base)];
  if (t.max_pos < max_pos) {
    int cap = max_pos > 2 * t.max_pos ? max_pos : 2 * t.max_pos;
    cap = (cap + 1023) / 1024 * 1024;
    const int half = d / 2;
    std::vector<float> c((size_t)cap * half), s((size_t)cap * half);
    for (int i = 0; i < half; ++i) {
      const double f = std::pow(base, -2.0 * i / d);
      for (int p = 0; p < cap; ++p) {
        const double th = (double)p * f;
        c[(size_t)p * half + i] = (float)std::cos(th);
        s[(size_t)p * half + i] = (float)std::sin(th);
      }
    }
    float *dc = nullptr, *ds = nullptr;
    SRP_HIP(hipMalloc(&dc, c.size() * sizeof(float)));
    SRP_HIP(hipMalloc(&ds, s.size() * sizeof(float)));
    SRP_HIP(hipMemcpy(dc, c.data(), c.size() * sizeof(float), hipMemcpyHostToDevice));
    SRP_HIP(hipMemcpy(ds, s.data(), s.size() * sizeof(float), hipMemcpyHostToDevice));
    if (t.cos_t) {
      g_retired.push_back(t.cos_t);
      g_retired.push_back(t.sin_t);
    }
    t.cos_t = dc;
    t.sin_t = ds;
    t.max_pos = cap;
  }
  *out = RopeTable{t.cos_t, t.sin_t, d / 2, t.max_pos};
  return SRP_OK;
}

// ------------------------------------------------------------------------- //
// stage timing: hipEvents recorded on the caller's stream between the launch
// stages of srp_fuse_layer, one row of events per call, up to a capacity
// ------------------------------------------------------------------------- //
constexpr int kStages = 6;
const char *kStageNames[kStages] = {"prepare", "kv_proj", "select", "scatter", "q_proj", "attention"};
struct Profile {
  bool on = false;
  int cap = 0, used = 0;
  std::vector<hipEvent_t> ev;  // cap * (kStages + 1)
};
std::mutex g_pmu;
Profile g_prof;

// Records event `i` of the current call if profiling is on.
struct StageMarks {
  hipStream_t s;
  hipEvent_t *row = nullptr;
  explicit StageMarks(hipStream_t st) : s(st) {
    std::lock_guard<std::mutex> lk(g_pmu);
    if (g_prof.on && g_prof.used < g_prof.cap) row = &g_prof.ev[(size_t)g_prof.used++ * (kStages + 1)];
  }
  void mark(int i) {
    if (row) (void)hipEventRecord(row[i], s);
  }
};

// ------------------------------------------------------------------------- //
// argument checks
// ------------------------------------------------------------------------- //
int check_dims(const srp_dims *d) {
  if (!d) return fail(SRP_E_INVALID, "dims is NULL");
  if (d->dtype != SRP_F32 && d->dtype != SRP_BF16) return fail(SRP_E_INVALID, "dtype %d unknown", d->dtype);
  if (d->hidden <= 0 || d->hidden % 64) return fail(SRP_E_INVALID, "hidden %d must be a positive multiple of 64", d->hidden);
  if (d->n_kv_heads <= 0 || d->n_heads <= 0 || d->n_heads % d->n_kv_heads)
    return fail(SRP_E_INVALID, "n_heads %d must be a positive multiple of n_kv_heads %d", d->n_heads, d->n_kv_heads);
  if (d->n_heads / d->n_kv_heads > 8) return fail(SRP_E_UNSUPPORTED, "more than 8 query heads per KV head");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(SRP_E_UNSUPPORTED, "head_dim %d (64 or 128 supported)", d->head_dim);
  if (!(d->rope_base > 1.0) || !std::isfinite(d->rope_base)) return fail(SRP_E_INVALID, "rope_base must be > 1");
  return SRP_OK;
}

int check_batch(const srp_batch *b) {
  if (!b) return fail(SRP_E_INVALID, "batch is NULL");
  if (b->n_req < 1 || b->n_chunks < 1 || b->total_rows < 0 || b->max_req_rows < 0 || b->max_position < 1)
    return fail(SRP_E_INVALID, "batch sizes out of range (n_req %d, n_chunks %d, rows %d, max_req_rows %d, max_position %d)",
                b->n_req, b->n_chunks, b->total_rows, b->max_req_rows, b->max_position);
  if (b->total_rows > 0 && b->max_req_rows < 1) return fail(SRP_E_INVALID, "max_req_rows must be >= 1");
  if (!b->req_offsets || !b->chunk_offsets || !b->chunk_src_pos || (b->total_rows > 0 && !b->positions))
    return fail(SRP_E_INVALID, "batch device arrays must not be NULL");
  if (b->block_rows < 0 || b->block_rows > 4096) return fail(SRP_E_INVALID, "block_rows must lie in [0, 4096]");
  if (b->block_rows > 0 && (!b->seg_block || !b->block_table))
    return fail(SRP_E_INVALID, "a paged cache needs seg_block and block_table");
  return SRP_OK;
}

int check_select(const srp_select *s) {
  if (!s) return fail(SRP_E_INVALID, "select is NULL");
  if (s->mode != SRP_SEL_TOPK && s->mode != SRP_SEL_GIVEN && s->mode != SRP_SEL_SCORES)
    return fail(SRP_E_INVALID, "selection mode %d unknown", s->mode);
  if (!(s->ratio >= 0.0 && s->ratio <= 1.0)) return fail(SRP_E_INVALID, "ratio must lie in [0, 1]");
  if (s->dev_mode != SRP_DEV_KV && s->dev_mode != SRP_DEV_V) return fail(SRP_E_INVALID, "dev_mode %d unknown", s->dev_mode);
  if (s->k_rule != SRP_K_ROUND && s->k_rule != SRP_K_CEIL) return fail(SRP_E_INVALID, "k_rule %d unknown", s->k_rule);
  if (s->fresh_all != 0 && s->fresh_all != 1) return fail(SRP_E_INVALID, "fresh_all must be 0 or 1");
  if (s->window < 0) return fail(SRP_E_INVALID, "window must be >= 0");
  if (s->window > 0) {
    if (s->tau < 1 || s->tau > s->window) return fail(SRP_E_INVALID, "tau must lie in [1, window]");
    if (s->cand) return fail(SRP_E_INVALID, "grouping scans every cached row: cand must be NULL");
  }
  if (s->cand && !s->cand_offsets) return fail(SRP_E_INVALID, "cand needs cand_offsets");
  if (s->mode == SRP_SEL_GIVEN && !s->cand) return fail(SRP_E_INVALID, "SRP_SEL_GIVEN needs a candidate list");
  if ((s->mode == SRP_SEL_SCORES) != (s->scores != nullptr))
    return fail(SRP_E_INVALID, "scores are given exactly in SRP_SEL_SCORES mode");
  if (s->span_max != 0) {
    if (s->mode != SRP_SEL_SCORES) return fail(SRP_E_INVALID, "span completion needs SRP_SEL_SCORES");
    if (s->span_max < 1 || s->span_max > 1024) return fail(SRP_E_INVALID, "span_max must lie in [1, 1024]");
    if (s->window > 0) return fail(SRP_E_INVALID, "span completion and window grouping exclude each other");
    if (s->cand) return fail(SRP_E_INVALID, "span completion scans every cached row: cand must be NULL");
    if (!(s->tau_smooth >= 0.0)) return fail(SRP_E_INVALID, "tau_smooth must be >= 0");
    if (!(s->tau_cover >= 0.0 && s->tau_cover <= 1.0)) return fail(SRP_E_INVALID, "tau_cover must lie in [0, 1]");
  }
  if (s->cap_ratio != 0.0) {
    if (s->span_max == 0) return fail(SRP_E_INVALID, "cap_ratio applies to span completion only");
    if (!(s->cap_ratio >= s->ratio && s->cap_ratio <= 1.0))
      return fail(SRP_E_INVALID, "cap_ratio must lie in [ratio, 1]");
  }
  return SRP_OK;
}

// Checks that depend on both the batch and the selection.
int check_select_batch(const srp_batch *b, const srp_select *s) {
  if (s->mode == SRP_SEL_SCORES && b->max_req_rows > kLdsEntries)
    return fail(SRP_E_UNSUPPORTED, "SRP_SEL_SCORES handles requests of at most %d rows (max_req_rows %d)",
                kLdsEntries, b->max_req_rows);
  return SRP_OK;
}

#define CHECK(x)            \
  do {                      \
    int rc_ = (x);          \
    if (rc_ != SRP_OK) return rc_; \
  } while (0)

}  // namespace

extern "C" {

const char *srp_last_error(void) { return g_err.c_str(); }
const char *srp_version(void) { return "libsrp 0.1 gfx950"; }

int srp_workspace_size(const srp_dims *dims, const srp_batch *batch, const srp_select *sel, size_t *bytes) {
  CHECK(check_dims(dims));
  CHECK(check_batch(batch));
  CHECK(check_select(sel));
  CHECK(check_select_batch(batch, sel));
  if (!bytes) return fail(SRP_E_INVALID, "bytes is NULL");
  *bytes = carve(*dims, *batch, nullptr).bytes;
  return SRP_OK;
}

}  // extern "C"

namespace {

// Argument checks of srp_fuse_layer that do not involve the workspace.
int check_fuse_args(const srp_dims *dims, const srp_batch *batch, const srp_select *sel,
                    const void *hidden, const void *w_qkv, const void *k_cache, const void *v_cache,
                    const int32_t *sel_idx, const int32_t *sel_offsets, const void *attn_out) {
  CHECK(check_dims(dims));
  CHECK(check_batch(batch));
  CHECK(check_select(sel));
  CHECK(check_select_batch(batch, sel));
  if (batch->total_rows > 0 && (!hidden || !w_qkv || !k_cache || !v_cache || !sel_idx || !attn_out))
    return fail(SRP_E_INVALID, "tensor arguments must not be NULL");
  if (!sel_offsets) return fail(SRP_E_INVALID, "sel_offsets must not be NULL");
  return SRP_OK;
}

// The launch sequence of one fused layer on a carved workspace and a rotary table.
int fuse_layer_launch(const srp_dims &d, const srp_batch &b, const srp_select *sel, const void *hidden,
                      const void *w_qkv, void *k_cache, void *v_cache, int32_t *sel_idx,
                      int32_t *sel_offsets, void *attn_out, float *dev_out, const Workspace &w,
                      const RopeTable &rt, hipStream_t s) {
  const int T = b.total_rows;
  const int kvd = d.n_kv_heads * d.head_dim, qd = d.n_heads * d.head_dim;
  const size_t es = d.dtype == SRP_BF16 ? 2 : 4;

  SelectArgs sa{};
  sa.n_req = b.n_req;
  sa.T = T;
  sa.max_req_rows = b.max_req_rows;
  sa.req_offsets = b.req_offsets;
  sa.chunk_offsets = b.chunk_offsets;
  sa.chunk_src_pos = b.chunk_src_pos;
  sa.positions = b.positions;
  sa.n_chunks = b.n_chunks;
  sa.mode = sel->mode;
  sa.window = sel->window;
  sa.tau = sel->tau;
  sa.dev_mode = sel->dev_mode;
  sa.ratio = sel->ratio;
  sa.cand = sel->cand;
  sa.cand_offsets = sel->cand_offsets;
  sa.nkv = d.n_kv_heads;
  sa.dev_out = dev_out;
  sa.tile_rows = attn_tile_rows(d.dtype, d.n_heads, d.n_kv_heads);
  sa.k_ceil = sel->k_rule == SRP_K_CEIL;
  sa.scores = sel->scores;
  sa.span_max = sel->span_max;
  sa.tau_smooth = sel->tau_smooth;
  sa.tau_cover = sel->tau_cover;
  sa.cap_ratio = sel->cap_ratio;
  sa.fresh_all = sel->fresh_all;
  sa.block_rows = b.block_rows;
  sa.seg_block = b.seg_block;
  sa.block_table = b.block_table;
  // with external scores the rows are chosen first and then handled as a given list
  const bool by_scores = sel->mode == SRP_SEL_SCORES;
  sa.listed = sel->cand != nullptr || by_scores;
  SelectArgs sd = sa;
  if (by_scores) {
    sd.mode = SRP_SEL_GIVEN;
    sd.window = 0;
    sd.span_max = 0;
  }
  // V-only deviation needs only the V projection of the candidates: their fresh
  // keys are dropped unless selected, so K is projected for the selection alone,
  // together with Q (CacheClip paper's account of CacheBlend: value matrices)
  const bool v_only = sel->mode == SRP_SEL_TOPK && sel->dev_mode == SRP_DEV_V && !sel->fresh_all;
  sd.v_only = v_only;

  // 1. row metadata; candidate list, the choice by scores, and the recomputed rows
  //    R when they are listed
  StageMarks marks(s);
  marks.mark(0);
  SRP_HIP(launch_prepare(sa, w, s));
  // 2. positional recovery of cached rows outside R (inside R the projection
  //    epilogue rotates them next to the deviation; with V-only deviation, of
  //    every cached row)
  if ((sa.listed || v_only) && T > 0)
    SRP_HIP(launch_rerotate(d.dtype, T, d.n_kv_heads, d.head_dim, w.row_delta, w.row_slot,
                            PagedMap{b.block_rows, b.seg_block, b.block_table}, b.chunk_offsets,
                            b.n_chunks, b.chunk_src_pos, b.positions, v_only ? nullptr : w.rowflag, rt,
                            k_cache, s));
  // 3. K/V projection of R with the rotation / deviation epilogue (V alone with
  //    V-only deviation)
  GemmArgs g{};
  g.dtype = d.dtype;
  g.A = hidden;
  g.K = d.hidden;
  g.a_rows = sa.listed ? w.rlist : nullptr;
  g.M_host = T;
  g.M_dev = sa.listed ? w.ctr + kCtrREntries : nullptr;
  g.M_cap = T;
  g.B = (const char *)w_qkv + (size_t)(v_only ? qd + kvd : qd) * d.hidden * es;
  g.N = v_only ? kvd : 2 * kvd;
  g.mode = v_only ? EPI_V : EPI_KV;
  g.nh = d.n_heads;
  g.nkv = d.n_kv_heads;
  g.d = d.head_dim;
  g.positions = b.positions;
  g.row_delta = w.row_delta;
  g.rope = rt;
  g.k_cache = k_cache;
  g.v_cache = v_cache;
  g.fresh = w.fresh_kv;
  g.dev_part = w.dev_part;
  g.row_slot = w.row_slot;
  g.part = w.gemm_part;
  g.part_cap = w.gemm_part ? w.gemm_parts : 0;
  marks.mark(1);
  SRP_HIP(launch_gemm(g, s));
  marks.mark(2);
  // 4. top-k / grouping per request, CSR offsets, attention tiles
  SRP_HIP(launch_select(sd, w, sel_offsets, s));
  marks.mark(3);
  // 5. sel_idx and the scatter of fresh K/V into the cache
  SRP_HIP(launch_compact_scatter(sd, w, d.dtype, kvd, sel_idx, sel_offsets, k_cache, v_cache, s));
  // a paged cache is gathered in row order for the attention's key tiles (and, in
  // fp32, its value rows); the bf16 value transpose reads the pool rows itself
  const void *k_att = k_cache, *v_att = v_cache;
  if (w.row_slot && T > 0 && d.dtype != SRP_BF16) {
    SRP_HIP(launch_gather_rows(T, (size_t)kvd * es, w.row_slot, v_cache, w.v_lin, s));
    v_att = w.v_lin;
  }
  marks.mark(4);
  // 6. Q projection of the selected rows (with V-only deviation also their fresh
  //    keys, straight into the cache)
  GemmArgs gq = g;
  gq.a_rows = sel_idx;
  gq.M_dev = w.ctr + kCtrTotalSel;
  gq.B = w_qkv;
  gq.N = v_only ? qd + kvd : qd;
  gq.mode = v_only ? EPI_QK : EPI_Q;
  gq.q_out = w.q;
  // bf16 attention works in base 2 on pre-scaled queries; the fp32 kernel scales itself
  gq.q_scale = d.dtype == SRP_BF16 ? (float)(1.4426950408889634 / std::sqrt((double)d.head_dim)) : 1.0f;
  if (d.dtype == SRP_BF16 && T > 0) {
    // the work-groups the projection leaves idle transpose the fused V (the
    // selection's finalize zeroed the chunk counter)
    gq.vt_src = v_cache;
    gq.vt_slot = w.row_slot;
    gq.vt_dst = w.vt;
    gq.vt_T = T;
    gq.vt_stride = vt_stride(T);
    gq.vt_ctr = w.ctr + kCtrVtChunks;
  }
  SRP_HIP(launch_gemm(gq, s));
  if (w.row_slot && T > 0) {
    // the fused keys are final only now
    SRP_HIP(launch_gather_rows(T, (size_t)kvd * es, w.row_slot, k_cache, w.k_lin, s));
    k_att = w.k_lin;
  }
  marks.mark(5);
  // 7. attention of the selected rows over the fused cache
  AttnArgs aa{};
  aa.dtype = d.dtype;
  aa.nh = d.n_heads;
  aa.nkv = d.n_kv_heads;
  aa.d = d.head_dim;
  aa.q = w.q;
  aa.sel_idx = sel_idx;
  aa.req_offsets = b.req_offsets;
  aa.tiles = w.tiles;
  aa.n_tiles = w.ctr + kCtrTiles;
  aa.max_tiles = max_attn_tiles(T, b.n_req);
  aa.k_cache = k_att;
  aa.v_cache = v_att;
  aa.vt = w.vt;
  aa.vt_stride = vt_stride(T);
  aa.total_rows = T;
  aa.out = attn_out;
  if (T > 0) SRP_HIP(launch_attention(aa, s));
  marks.mark(6);
  return SRP_OK;
}

}  // namespace

extern "C" {

int srp_fuse_layer(const srp_dims *dims, const srp_batch *batch, const srp_select *sel,
                   const void *hidden, const void *w_qkv, void *k_cache, void *v_cache,
                   int32_t *sel_idx, int32_t *sel_offsets, void *attn_out, float *dev_out,
                   void *workspace, size_t workspace_bytes, srp_stream_t stream) {
  g_err.clear();
  CHECK(check_fuse_args(dims, batch, sel, hidden, w_qkv, k_cache, v_cache, sel_idx, sel_offsets, attn_out));
  const size_t need = carve(*dims, *batch, nullptr).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(SRP_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  RopeTable rt;
  CHECK(get_table(dims->head_dim, dims->rope_base, batch->max_position, &rt));
  return fuse_layer_launch(*dims, *batch, sel, hidden, w_qkv, k_cache, v_cache, sel_idx, sel_offsets,
                           attn_out, dev_out, carve(*dims, *batch, (char *)workspace), rt,
                           (hipStream_t)stream);
}

}  // extern "C"

// ------------------------------------------------------------------------- //
// no-allocation variant: the workspace and the rotary table live in `scratch`, a
// file-scope device array of kScratchBytes that every GPU the library runs on
// holds until the process ends. Host code never uses the array's name as an
// address (in host code it only stands in for the symbol): its device address on
// each device comes from hipGetSymbolAddress on the first call there.
// ------------------------------------------------------------------------- //
namespace {

constexpr size_t kScratchBytes = (size_t)128 << 20;
// split-K partial-tile slots the variant carves (4 MiB; the workspace variant: 256)
constexpr int kScratchParts = 16;
constexpr int kMaxDevices = 64;

struct ScratchDev {
  char *ptr = nullptr;      // device address of `scratch` on this device
  int table_d = 0;          // the rotary table at the front of the array: head dim,
  double table_base = 0.0;  // base
  int table_cap = 0;        // and positions covered (0: none built)
};
std::mutex g_smu;
ScratchDev g_sdev[kMaxDevices];

// cos / sin of p * base^(-2i/d) for p < n_pos, i < d/2, evaluated in double and
// rounded to float (the same expressions as the host-built tables).
__global__ void rope_table_kernel(float *cos_t, float *sin_t, int half, int d, double base, int n_pos) {
  const long n = (long)n_pos * half;
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (long)gridDim.x * blockDim.x) {
    const int p = (int)(t / half), i = (int)(t - (long)p * half);
    const double f = pow(base, -2.0 * i / d);
    const double th = (double)p * f;
    cos_t[t] = (float)cos(th);
    sin_t[t] = (float)sin(th);
  }
}

size_t table_bytes(int d, int cap) { return align_up((size_t)cap * (d / 2) * sizeof(float), 256) * 2; }

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

extern "C" {

int srp_fuse_layer_noalloc(const srp_dims *dims, const srp_batch *batch, const srp_select *sel,
                           const void *hidden, const void *w_qkv, void *k_cache, void *v_cache,
                           int32_t *sel_idx, int32_t *sel_offsets, void *attn_out, float *dev_out,
                           srp_stream_t stream) {
  g_err.clear();
  CHECK(check_fuse_args(dims, batch, sel, hidden, w_qkv, k_cache, v_cache, sel_idx, sel_offsets, attn_out));
  const srp_dims &d = *dims;
  const srp_batch &b = *batch;
  hipStream_t s = (hipStream_t)stream;
  // host-checkable size limit first: the table of this call's positions plus the
  // workspace (a table kept from an earlier call may be larger, checked below)
  const int cap0 = (b.max_position + 1023) / 1024 * 1024;
  const size_t ws_bytes = carve(d, b, nullptr, kScratchParts).bytes;
  if (table_bytes(d.head_dim, cap0) + ws_bytes > kScratchBytes)
    return fail(SRP_E_WORKSPACE,
                "this layer needs %zu bytes of scratch; srp_fuse_layer_noalloc has %zu (use srp_fuse_layer with a workspace)",
                table_bytes(d.head_dim, cap0) + ws_bytes, kScratchBytes);
  int dev = 0;
  SRP_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(SRP_E_UNSUPPORTED, "device %d beyond the %d the variant tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_smu);
  ScratchDev &sd = g_sdev[dev];
  if (!sd.ptr) {
    // once per device, with that device current
    void *p = nullptr;
    SRP_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(SRP_E_HIP, "hipGetSymbolAddress returned no address for the scratch array");
    sd.ptr = (char *)p;
  }
  // the table is rebuilt only when this call needs another one (or more positions)
  const bool rebuild = sd.table_cap == 0 || sd.table_d != d.head_dim || sd.table_base != d.rope_base ||
                       sd.table_cap < b.max_position;
  int cap = rebuild ? cap0 : sd.table_cap;
  // a larger kept table that leaves too little room is rebuilt at this call's size
  if (!rebuild && table_bytes(d.head_dim, cap) + ws_bytes > kScratchBytes) cap = cap0;
  const bool build = rebuild || cap != sd.table_cap;
  const size_t tb = table_bytes(d.head_dim, cap);
  const int half = d.head_dim / 2;
  float *cos_t = (float *)sd.ptr, *sin_t = (float *)(sd.ptr + tb / 2);
  if (build) {
    const long n = (long)cap * half;
    const unsigned grid = (unsigned)std::min<long>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(rope_table_kernel, dim3(grid), dim3(256), 0, s, cos_t, sin_t, half, d.head_dim,
                       d.rope_base, cap);
    SRP_HIP(hipGetLastError());
    sd.table_d = d.head_dim;
    sd.table_base = d.rope_base;
    sd.table_cap = cap;
  }
  const RopeTable rt{cos_t, sin_t, half, cap};
  return fuse_layer_launch(d, b, sel, hidden, w_qkv, k_cache, v_cache, sel_idx, sel_offsets, attn_out,
                           dev_out, carve(d, b, sd.ptr + tb, kScratchParts), rt, s);
}

int srp_profile_begin(int32_t max_calls) {
  g_err.clear();
  if (max_calls < 1) return fail(SRP_E_INVALID, "max_calls must be >= 1");
  std::lock_guard<std::mutex> lk(g_pmu);
  const size_t need = (size_t)max_calls * (kStages + 1);
  while (g_prof.ev.size() < need) {
    hipEvent_t e;
    SRP_HIP(hipEventCreate(&e));
    g_prof.ev.push_back(e);
  }
  g_prof.cap = max_calls;
  g_prof.used = 0;
  g_prof.on = true;
  return SRP_OK;
}

int srp_profile_end(float *ms, int32_t max_calls, int32_t *n_calls) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_pmu);
  if (!g_prof.on) return fail(SRP_E_INVALID, "profiling was not started");
  g_prof.on = false;
  const int n = g_prof.used < max_calls ? g_prof.used : max_calls;
  if (n_calls) *n_calls = n;
  for (int c = 0; c < n; ++c) {
    hipEvent_t *row = &g_prof.ev[(size_t)c * (kStages + 1)];
    SRP_HIP(hipEventSynchronize(row[kStages]));
    for (int i = 0; i < kStages; ++i)
      SRP_HIP(hipEventElapsedTime(&ms[(size_t)c * kStages + i], row[i], row[i + 1]));
  }
  return SRP_OK;
}

const char *srp_profile_stage_name(int32_t i) { return (i >= 0 && i < kStages) ? kStageNames[i] : ""; }

int srp_encode_kv(const srp_dims *dims, int32_t n_rows, int32_t max_position, const void *hidden,
                  const void *w_qkv, const int32_t *positions, void *k_out, void *v_out,
                  srp_stream_t stream) {
  g_err.clear();
  CHECK(check_dims(dims));
  if (n_rows < 0 || max_position < 1) return fail(SRP_E_INVALID, "n_rows / max_position out of range");
  if (n_rows == 0) return SRP_OK;
  if (!hidden || !w_qkv || !positions || !k_out || !v_out) return fail(SRP_E_INVALID, "NULL tensor argument");
  const srp_dims &d = *dims;
  RopeTable rt;
  CHECK(get_table(d.head_dim, d.rope_base, max_position, &rt));
  const size_t es = d.dtype == SRP_BF16 ? 2 : 4;
  GemmArgs g{};
  g.dtype = d.dtype;
  g.A = hidden;
  g.K = d.hidden;
  g.M_host = n_rows;
  g.M_cap = n_rows;
  g.B = (const char *)w_qkv + (size_t)d.n_heads * d.head_dim * d.hidden * es;
  g.N = 2 * d.n_kv_heads * d.head_dim;
  g.mode = EPI_ENC;
  g.nh = d.n_heads;
  g.nkv = d.n_kv_heads;
  g.d = d.head_dim;
  g.positions = positions;
  g.rope = rt;
  g.k_cache = k_out;
  g.v_cache = v_out;
  SRP_HIP(launch_gemm(g, (hipStream_t)stream));
  return SRP_OK;
}

int srp_rerotate_kv(const srp_dims *dims, const srp_batch *batch, void *k_cache, srp_stream_t stream) {
  g_err.clear();
  CHECK(check_dims(dims));
  CHECK(check_batch(batch));
  if (batch->total_rows == 0) return SRP_OK;
  if (!k_cache) return fail(SRP_E_INVALID, "k_cache is NULL");
  RopeTable rt;
  CHECK(get_table(dims->head_dim, dims->rope_base, batch->max_position, &rt));
  SRP_HIP(launch_rerotate(dims->dtype, batch->total_rows, dims->n_kv_heads, dims->head_dim, nullptr, nullptr,
                          PagedMap{batch->block_rows, batch->seg_block, batch->block_table},
                          batch->chunk_offsets, batch->n_chunks, batch->chunk_src_pos,
                          batch->positions, nullptr, rt, k_cache, (hipStream_t)stream));
  return SRP_OK;
}

int srp_residual_rmsnorm(const srp_dims *dims, void *hidden, const void *attn_out,
                         const int32_t *sel_idx, const int32_t *sel_offsets, int32_t n_req,
                         int32_t sel_capacity, float eps, srp_stream_t stream) {
  g_err.clear();
  CHECK(check_dims(dims));
  if (dims->n_heads * dims->head_dim != dims->hidden)
    return fail(SRP_E_INVALID, "residual needs n_heads * head_dim == hidden");
  if (n_req < 1 || sel_capacity < 0 || !(eps >= 0.f)) return fail(SRP_E_INVALID, "n_req / sel_capacity / eps out of range");
  if (sel_capacity == 0) return SRP_OK;
  if (!hidden || !attn_out || !sel_idx || !sel_offsets) return fail(SRP_E_INVALID, "NULL tensor argument");
  SRP_HIP(launch_residual_rmsnorm(dims->dtype, dims->hidden, hidden, attn_out, sel_idx,
                                  sel_offsets + n_req, sel_capacity, eps, (hipStream_t)stream));
  return SRP_OK;
}

// ------------------------------------------------------------------------- //
// stack executor: cache loads on a copy stream, layers on the compute stream
// ------------------------------------------------------------------------- //
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int srp_stack_workspace_size(const srp_dims *dims, const srp_batch *batch, const srp_select *first,
                             size_t *bytes) {
  g_err.clear();
  if (!bytes) return fail(SRP_E_INVALID, "bytes is NULL");
  size_t layer = 0;
  CHECK(srp_workspace_size(dims, batch, first, &layer));
  *bytes = align256(layer) + align256((size_t)(batch->total_rows > 0 ? batch->total_rows : 1) * 4) +
           align256((size_t)(batch->n_req + 1) * 4);
  return SRP_OK;
}

// A second copy stream per device for the stack executor's value loads (created on
// first use with the default priority, kept until the process ends): with the keys
// on the caller's copy stream and the values on this one, one copy engine's idle
// time between transfers overlaps the other's transfer.
static hipError_t value_copy_stream(hipStream_t *out) {
  static std::mutex mu;
  static std::map<int, hipStream_t> streams;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = streams.find(dev);
  if (it == streams.end()) {
    hipStream_t st;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    it = streams.emplace(dev, st).first;
  }
  *out = it->second;
  return hipSuccess;
}

int srp_fuse_stack(const srp_dims *dims, const srp_batch *batch, const srp_select *first,
                   int32_t n_layers, const srp_layer *layers, void *hidden, float rms_eps,
                   int32_t *sel_idx, int32_t *sel_offsets, void *attn_out, void *workspace,
                   size_t workspace_bytes, srp_stream_t stream, srp_stream_t copy_stream) {
  g_err.clear();
  CHECK(check_dims(dims));
  CHECK(check_batch(batch));
  CHECK(check_select(first));
  CHECK(check_select_batch(batch, first));
  if (n_layers < 1 || !layers) return fail(SRP_E_INVALID, "n_layers must be >= 1 with a layer array");
  if (dims->n_heads * dims->head_dim != dims->hidden)
    return fail(SRP_E_INVALID, "the chain step needs n_heads * head_dim == hidden");
  if (!(rms_eps >= 0.f)) return fail(SRP_E_INVALID, "rms_eps must be >= 0");
  const srp_batch &b = *batch;
  const int T = b.total_rows;
  for (int l = 0; l < n_layers; ++l) {
    const srp_layer &L = layers[l];
    if (!(L.ratio >= 0.0 && L.ratio <= 1.0)) return fail(SRP_E_INVALID, "layer %d: ratio must lie in [0, 1]", l);
    if (l > 0 && L.mode != SRP_SEL_TOPK && L.mode != SRP_SEL_GIVEN)
      return fail(SRP_E_INVALID, "layer %d: mode must be SRP_SEL_TOPK or SRP_SEL_GIVEN", l);
    if ((L.k_host == nullptr) != (L.v_host == nullptr))
      return fail(SRP_E_INVALID, "layer %d: k_host and v_host go together", l);
    if (T > 0 && (!L.w_qkv || !L.k_cache || !L.v_cache))
      return fail(SRP_E_INVALID, "layer %d: NULL device tensor", l);
  }
  if (T > 0 && (!hidden || !sel_idx || !attn_out)) return fail(SRP_E_INVALID, "tensor arguments must not be NULL");
  if (!sel_offsets) return fail(SRP_E_INVALID, "sel_offsets must not be NULL");
  size_t need = 0, layer_ws = 0;
  CHECK(srp_stack_workspace_size(dims, batch, first, &need));
  CHECK(srp_workspace_size(dims, batch, first, &layer_ws));
  if (!workspace || workspace_bytes < need)
    return fail(SRP_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  char *ws = (char *)workspace;
  int32_t *cand_idx = (int32_t *)(ws + align256(layer_ws));
  int32_t *cand_off = (int32_t *)((char *)cand_idx + align256((size_t)(T > 0 ? T : 1) * 4));
  hipStream_t s = (hipStream_t)stream, cs = (hipStream_t)copy_stream;
  const size_t cache_bytes = (size_t)T * dims->n_kv_heads * dims->head_dim * (dims->dtype == SRP_BF16 ? 2 : 4);

  // one event per loaded layer and copy stream, created for this call (concurrent
  // calls never share one) and released once its wait is enqueued. The copy
  // streams wait for nothing: a copy stream made to wait for work still pending on
  // the compute stream can stall the host inside hipMemcpyAsync for milliseconds
  // (measured), which idles the GPU; the caller keeps the destinations free instead.
  std::vector<hipEvent_t> ev(n_layers, nullptr), ev_v(n_layers, nullptr);
  auto release = [&]() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : ev_v)
      if (e) (void)hipEventDestroy(e);
  };
  bool loads = false;
  for (int l = 0; l < n_layers; ++l) loads |= layers[l].k_host != nullptr;
  if (loads && b.block_rows > 0)
    return fail(SRP_E_UNSUPPORTED, "host loads fill contiguous caches (block_rows must be 0)");
  // on a side stream the values go to a second copy stream; in line (cs == s)
  // both copies stay on the compute stream
  hipStream_t vs = cs;
  if (loads && cache_bytes > 0 && cs != s) {
    hipError_t e = value_copy_stream(&vs);
    if (e != hipSuccess) return fail(SRP_E_HIP, "the value copy stream: %s", hipGetErrorString(e));
  }
  for (int l = 0; l < n_layers; ++l) {
    if (!layers[l].k_host || cache_bytes == 0) continue;
    hipError_t e = hipEventCreateWithFlags(&ev[l], hipEventDisableTiming);
    if (e == hipSuccess && vs != cs) e = hipEventCreateWithFlags(&ev_v[l], hipEventDisableTiming);
    if (e == hipSuccess) e = hipMemcpyAsync(layers[l].k_cache, layers[l].k_host, cache_bytes, hipMemcpyHostToDevice, cs);
    if (e == hipSuccess) e = hipMemcpyAsync(layers[l].v_cache, layers[l].v_host, cache_bytes, hipMemcpyHostToDevice, vs);
    if (e == hipSuccess) e = hipEventRecord(ev[l], cs);
    if (e == hipSuccess && ev_v[l]) e = hipEventRecord(ev_v[l], vs);
    if (e != hipSuccess) {
      release();
      return fail(SRP_E_HIP, "loading layer %d: %s", l, hipGetErrorString(e));
    }
  }
  int rc = SRP_OK;
  for (int l = 0; l < n_layers && rc == SRP_OK; ++l) {
    if (ev[l]) {
      hipError_t e = hipStreamWaitEvent(s, ev[l], 0);
      if (e == hipSuccess && ev_v[l]) e = hipStreamWaitEvent(s, ev_v[l], 0);
      if (e != hipSuccess) {
        rc = fail(SRP_E_HIP, "waiting for layer %d: %s", l, hipGetErrorString(e));
        break;
      }
    }
    srp_select sl = *first;
    sl.ratio = layers[l].ratio;
    if (l > 0) {
      sl = srp_select{};
      sl.mode = layers[l].mode;
      sl.ratio = layers[l].ratio;
      sl.dev_mode = first->dev_mode;
      sl.k_rule = first->k_rule;
      sl.fresh_all = first->fresh_all;
      sl.cand = cand_idx;
      sl.cand_offsets = cand_off;
    }
    rc = srp_fuse_layer(dims, batch, &sl, hidden, layers[l].w_qkv, layers[l].k_cache, layers[l].v_cache,
                        sel_idx, sel_offsets, attn_out, nullptr, workspace, layer_ws, stream);
    if (rc != SRP_OK) break;
    if (l + 1 < n_layers) {
      // the next layer's candidates: this layer's selection
      hipError_t e = hipMemcpyAsync(cand_idx, sel_idx, (size_t)(T > 0 ? T : 1) * 4, hipMemcpyDeviceToDevice, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(cand_off, sel_offsets, (size_t)(b.n_req + 1) * 4, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) {
        rc = fail(SRP_E_HIP, "carrying the selection of layer %d: %s", l, hipGetErrorString(e));
        break;
      }
    }
    rc = srp_residual_rmsnorm(dims, hidden, attn_out, sel_idx, sel_offsets, b.n_req, T, rms_eps, stream);
  }
  release();
  return rc;
}

int srp_controller_ratio(double full_layer_ms, double load_ms, double r_floor, double *ratio) {
  g_err.clear();
  if (!ratio) return fail(SRP_E_INVALID, "ratio is NULL");
  if (!(full_layer_ms > 0.0) || !(load_ms >= 0.0) || !(r_floor >= 0.0 && r_floor <= 1.0) ||
      !std::isfinite(full_layer_ms) || !std::isfinite(load_ms))
    return fail(SRP_E_INVALID, "need full_layer_ms > 0, load_ms >= 0 and 0 <= r_floor <= 1");
  const double r_equal = load_ms / full_layer_ms;
  const double r = r_equal > r_floor ? r_equal : r_floor;
  *ratio = r < 1.0 ? r : 1.0;
  return SRP_OK;
}

int srp_validate_batch(const srp_batch *batch, srp_stream_t stream) {
  g_err.clear();
  CHECK(check_batch(batch));
  const srp_batch &b = *batch;
  hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t> ro(b.n_req + 1), co(b.n_chunks + 1), cs(b.n_chunks), pos(b.total_rows);
  SRP_HIP(hipMemcpyAsync(ro.data(), b.req_offsets, ro.size() * 4, hipMemcpyDeviceToHost, s));
  SRP_HIP(hipMemcpyAsync(co.data(), b.chunk_offsets, co.size() * 4, hipMemcpyDeviceToHost, s));
  SRP_HIP(hipMemcpyAsync(cs.data(), b.chunk_src_pos, cs.size() * 4, hipMemcpyDeviceToHost, s));
  if (b.total_rows)
    SRP_HIP(hipMemcpyAsync(pos.data(), b.positions, pos.size() * 4, hipMemcpyDeviceToHost, s));
  SRP_HIP(hipStreamSynchronize(s));
  const int T = b.total_rows;
  if (ro[0] != 0 || ro[b.n_req] != T) return fail(SRP_E_BATCH, "req_offsets must run from 0 to total_rows");
  if (co[0] != 0 || co[b.n_chunks] != T) return fail(SRP_E_BATCH, "chunk_offsets must run from 0 to total_rows");
  for (int r = 0; r < b.n_req; ++r) {
    if (ro[r + 1] < ro[r]) return fail(SRP_E_BATCH, "req_offsets decrease at %d", r);
    if (ro[r + 1] - ro[r] > b.max_req_rows) return fail(SRP_E_BATCH, "request %d has more than max_req_rows rows", r);
    for (int j = ro[r] + 1; j < ro[r + 1]; ++j)
      if (pos[j] <= pos[j - 1]) return fail(SRP_E_BATCH, "positions not strictly increasing at row %d", j);
  }
  for (int j = 0; j < T; ++j)
    if (pos[j] < 0 || pos[j] >= b.max_position) return fail(SRP_E_BATCH, "position of row %d outside [0, max_position)", j);
  int r = 0;
  for (int c = 0; c < b.n_chunks; ++c) {
    if (co[c + 1] < co[c]) return fail(SRP_E_BATCH, "chunk_offsets decrease at %d", c);
    if (co[c + 1] == co[c]) continue;
    while (r < b.n_req && ro[r + 1] <= co[c]) ++r;
    if (r >= b.n_req || co[c] < ro[r] || co[c + 1] > ro[r + 1])
      return fail(SRP_E_BATCH, "segment %d crosses a request boundary", c);
    if (cs[c] < -1) return fail(SRP_E_BATCH, "chunk_src_pos[%d] < -1", c);
    if (cs[c] >= 0) {
      const long last = (long)cs[c] + (co[c + 1] - co[c]) - 1;
      if (last >= b.max_position) return fail(SRP_E_BATCH, "segment %d encoded past max_position", c);
      for (int j = co[c]; j < co[c + 1]; ++j) {
        const long delta = (long)pos[j] - (cs[c] + (j - co[c]));
        if (delta >= b.max_position || -delta >= b.max_position)
          return fail(SRP_E_BATCH, "|pos - src| of row %d reaches max_position", j);
      }
    }
  }
  if (b.block_rows > 0 && T > 0) {
    // paged cache: every row maps to its own pool row
    const int B = b.block_rows;
    std::vector<int32_t> sb(b.n_chunks);
    SRP_HIP(hipMemcpy(sb.data(), b.seg_block, sb.size() * 4, hipMemcpyDeviceToHost));
    long n_tab = 0;
    for (int c = 0; c < b.n_chunks; ++c) {
      const int len = co[c + 1] - co[c];
      if (len == 0) continue;
      if (sb[c] < 0) return fail(SRP_E_BATCH, "seg_block[%d] < 0", c);
      const long end = (long)sb[c] + (len + B - 1) / B;
      n_tab = end > n_tab ? end : n_tab;
    }
    std::vector<int32_t> tab(n_tab > 0 ? n_tab : 1);
    if (n_tab > 0) SRP_HIP(hipMemcpy(tab.data(), b.block_table, (size_t)n_tab * 4, hipMemcpyDeviceToHost));
    std::vector<long> rows;
    rows.reserve(T);
    for (int c = 0; c < b.n_chunks; ++c)
      for (int i = 0; i < co[c + 1] - co[c]; ++i) {
        const int blk = tab[sb[c] + i / B];
        if (blk < 0) return fail(SRP_E_BATCH, "negative block id for row %d", co[c] + i);
        rows.push_back((long)blk * B + i % B);
      }
    std::sort(rows.begin(), rows.end());
    for (size_t i = 1; i < rows.size(); ++i)
      if (rows[i] == rows[i - 1]) return fail(SRP_E_BATCH, "two rows map to pool row %ld", rows[i]);
  }
  return SRP_OK;
}

}  // extern "C"
