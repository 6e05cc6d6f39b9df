// Shared definitions of libsrp's HIP kernels and host code (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/srp.h"

namespace srp {

constexpr int kFresh = INT32_MIN;  // row_delta of a row without a cache
constexpr int kWave = 64;

// Per R-entry flags.
constexpr uint8_t kCand = 1;   // cached row that is scored (candidate)
constexpr uint8_t kFreshF = 2; // fresh row: always recomputed and selected
constexpr uint8_t kTop = 4;    // chosen by top-k
constexpr uint8_t kSel = 8;    // in the final selection

// Smallest attention query tile (selected rows per work-group); tiles are a
// multiple of it.
constexpr int kQT = 32;

// ------------------------------------------------------------------------- //
// bf16 storage
// ------------------------------------------------------------------------- //
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float ld(const float *p) { return *p; }
  __device__ static __forceinline__ void st(float *p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float ld(const uint16_t *p) { return bf2f(*p); }
  __device__ static __forceinline__ void st(uint16_t *p, float v) { *p = f2bf(v); }
};

// Load / store 4 consecutive elements as floats.
__device__ __forceinline__ void ld4(const float *p, float v[4]) {
  float4 t = *reinterpret_cast<const float4 *>(p);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void ld4(const uint16_t *p, float v[4]) {
  uint2 t = *reinterpret_cast<const uint2 *>(p);
  v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xffff0000u);
  v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xffff0000u);
}
__device__ __forceinline__ void st4(float *p, const float v[4]) {
  *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st4(uint16_t *p, const float v[4]) {
  uint2 t;
  t.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  t.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  *reinterpret_cast<uint2 *>(p) = t;
}

// ------------------------------------------------------------------------- //
// wave / block primitives (wave64)
// ------------------------------------------------------------------------- //
// Inclusive scan over the wave with DPP lane shifts (no LDS round trips):
// row_shr 1/2/4/8 scan each row of 16 lanes, row_bcast 15/31 carry the row
// totals into the rows above.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Exclusive scan over the block (blockDim.x a multiple of 64, <= 1024).
// `sh` needs 17 ints of LDS. Returns the exclusive prefix; *total = block sum.
__device__ __forceinline__ int block_excl_scan(int v, int *sh, int *total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) sh[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    // wave 0 scans the wave totals
    const int t = lane < nw ? sh[lane] : 0;
    const int ti = wave_incl_scan(t);
    if (lane < nw) sh[lane] = ti - t;
    if (lane == 63) sh[16] = ti;
  }
  __syncthreads();
  const int res = sh[wid] + inc - v;
  *total = sh[16];
  __syncthreads();
  return res;
}

__device__ __forceinline__ int block_sum(int v, int *sh) {
  int tot;
  block_excl_scan(v, sh, &tot);
  return tot;
}

// Largest i in [0, n) with a[i] <= x, for a non-decreasing a with a[0] <= x.
__device__ __forceinline__ int upper_index(const int32_t *a, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same for a wave whose lanes hold the table (t = a[lane] for lane < n, n <= 64,
// and a[0] <= x < a[n-1]): one ballot instead of dependent loads.
__device__ __forceinline__ int upper_index_lanes(int t, int n, int x) {
  const int lane = threadIdx.x & 63;
  return __popcll(__ballot(lane >= 1 && lane < n && t <= x));
}


// ------------------------------------------------------------------------- //
// rotary tables: cos/sin of p * base^(-2i/d), p < max_position, i < d/2,
// computed in fp64 on the host and stored as fp32 [max_position][d/2].
// ------------------------------------------------------------------------- //
struct RopeTable {
  const float *cos_t;
  const float *sin_t;
  int half;
  int max_pos;
};

// Rotate 4 rotation pairs (a[i], b[i]) = (x_i, x_{i+d/2}) by angle index p,
// p may be negative (rotation by -|p|).
__device__ __forceinline__ void rope4(float a[4], float b[4], const RopeTable &t, int p, int i0) {
  int ap = p < 0 ? -p : p;
  ap = ap < t.max_pos ? ap : t.max_pos - 1;  // never read past the table
  float c[4], s[4];
  ld4(t.cos_t + (size_t)ap * t.half + i0, c);
  ld4(t.sin_t + (size_t)ap * t.half + i0, s);
  const float sg = p < 0 ? -1.f : 1.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float sk = sg * s[k];
    float x = a[k], y = b[k];
    a[k] = x * c[k] - y * sk;
    b[k] = y * c[k] + x * sk;
  }
}

// ------------------------------------------------------------------------- //
// direct-to-LDS copies (gfx950 global_load_lds_dwordx4)
// ------------------------------------------------------------------------- //
typedef __attribute__((address_space(3))) void lds_void;

// One wave-wide direct-to-LDS copy: lane l's 16 bytes at src land at dst + 16 l
// (dst wave-uniform). Issued as inline asm so the compiler inserts no waits for
// it; the ring below waits for its copies explicitly (vmcnt) before a barrier.
// M0 is written here and used nowhere else by these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *src, char *dst) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_void *)dst;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(lds_addr)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with only the vector-memory counter constrained to <= n.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0): every LDS access this wave issued has completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// ------------------------------------------------------------------------- //
// workspace carve-up
// ------------------------------------------------------------------------- //
struct Workspace {
  int32_t *row_delta;  // [T] pos - src, kFresh for fresh rows
  int32_t *row_req;    // [T]
  uint8_t *rowflag;    // [T] candidate marks by row (candidate-list mode)
  int32_t *rlist;      // [T] R entry -> row (candidate-list mode)
  int32_t *roff;       // [n_req+1] R offsets (candidate-list mode)
  int32_t *blkcnt;     // compaction block counts; later per-request tile counts
  float *dev_part;     // [T][2 nkv] per-head squared-deviation partials
  void *fresh_kv;      // [T][2 kvdim] recomputed K (roped) and V, storage type
  uint32_t *keys;      // [T] fp32 bit patterns of squared deviations
  uint8_t *eflag;      // [T] per R-entry flags
  int32_t *seq_ent;    // [T] grouping: sequence slot -> entry
  int32_t *seq_pre;    // [T] grouping: prefix counts
  uint8_t *seq_flag;   // [T] grouping: top-k / passing-window flags
  int32_t *tsel_row;   // [T] selection per request, at the request's R offset
  int32_t *tsel_ent;   // [T]
  int32_t *sel_cnt;    // [n_req]
  int32_t *sel_ent;    // [T] compact: R entry of each selected row
  void *q;             // [T][qdim] roped queries of the selected rows
  void *vt;            // bf16: [nkv][d][vt_stride] fused V transposed for attention
  int32_t *tiles;      // [3 * max_tiles] attention tiles (first sel, count, req)
  int32_t *ctr;        // [16] device counters (see kCtr*)
  float *gemm_part;    // bf16: [kGemmParts][kGemmPartFloats] split-K partial tiles
  int32_t *row_slot;   // paged cache: [T] pool row of each batch row (else NULL)
  void *k_lin, *v_lin; // paged cache: [T][kvdim] fused K (and fp32 V) gathered in row order
  int gemm_parts;      // partial-tile slots at gemm_part (0: no split of the last round)
  size_t bytes;
};
// split-K partial tiles of the projection GEMMs' last round
constexpr int kGemmParts = 256;
constexpr size_t kGemmPartFloats = 256 * 256;
constexpr int kCtrTotalSel = 0;
constexpr int kCtrTiles = 1;
constexpr int kCtrREntries = 2;
constexpr int kCtrVtChunks = 3;  // V transpose chunks claimed (zeroed by the selection's finalize)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int blocks_per_req(int max_req_rows) { return (max_req_rows + 1023) / 1024 > 0 ? (max_req_rows + 1023) / 1024 : 1; }
// The selection's finalize may cut the longest attention tiles of an
// under-filled launch into halves of their queries, adding at most
// kAttnExtraTiles tiles; key blocks of the attention are kAttnBK rows.
constexpr int kAttnExtraTiles = 64;
constexpr int kAttnBK = 64;
inline int max_attn_tiles(int T, int n_req) { return T / kQT + n_req + 1 + kAttnExtraTiles; }
// Row stride of the transposed V copy: T rounded up to 64 plus one zeroed tile, so
// a key tile that starts inside the batch never reads past the copy.
inline int vt_stride(int T) { return (T + 63) / 64 * 64 + 64; }

// Chunks of the transposed V copy for the attention's DMA loads. Chunk (r0, g)
// covers keys r0..r0+63 of KV head g: row i of head g holds vt[g][i][j] =
// v[slot(j)][g][i] (slot(j) = row_slot[j], or j when row_slot is NULL); inside
// every 16-key group the keys are stored in the order 0-3, 8-11, 4-7, 12-15 (the
// PV operand's lane order); keys at or past T are zero. A work-group of NT
// threads does up to NCH chunks at once (n of them, chunk k at r0[k], g[k]): every
// global load is issued before the first LDS write, each thread writes two keys of
// one d per 32-bit LDS store, and each output 16 bytes comes from one LDS read.
// tile: NCH x 128 rows x kVtPitch u16 of LDS.
constexpr int kVtPitch = 72;  // u16 per LDS row (144 bytes: 16-byte aligned rows)
template <int NT, int NCH>
__device__ __forceinline__ void vt_chunks(int n, const int *r0, const int *g, int T, int D, int nkv,
                                          const uint16_t *v, const int32_t *row_slot, uint16_t *vt, int vts,
                                          uint16_t *tile) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, kvd = nkv * D, dch = D / 8;
  constexpr int ITEMS = 32 * 16 / NT > 0 ? (32 * 16 + NT - 1) / NT : 1;  // (key pair, d chunk) items per thread
  u32x4_t x[NCH][ITEMS][2];
#pragma unroll
  for (int k = 0; k < NCH; ++k)
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int c = tid + it * NT, kp = c & 31, dc = c >> 5;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        x[k][it][h] = u32x4_t{0, 0, 0, 0};
        const int row = k < n ? r0[k] + 2 * kp + h : T;
        if (dc < dch && row < T)
          x[k][it][h] =
              *reinterpret_cast<const u32x4_t *>(v + (size_t)(row_slot ? row_slot[row] : row) * kvd + g[k] * D + dc * 8);
      }
    }
#pragma unroll
  for (int k = 0; k < NCH; ++k)
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int c = tid + it * NT, kp = c & 31, dc = c >> 5;
      if (dc >= dch) continue;
      // stored position of key 2kp (bits 2 and 3 of its index swapped); key 2kp+1 follows
      const int key = 2 * kp, pos = (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
      uint16_t *t = tile + ((size_t)k * 128 + dc * 8) * kVtPitch + pos;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = x[k][it][0][i], b = x[k][it][1][i];
        *reinterpret_cast<uint32_t *>(t + (2 * i) * kVtPitch) = (a & 0xffffu) | (b << 16);
        *reinterpret_cast<uint32_t *>(t + (2 * i + 1) * kVtPitch) = (a >> 16) | (b & 0xffff0000u);
      }
    }
  __syncthreads();
  for (int k = 0; k < n; ++k)
    for (int c = tid; c < D * 8; c += NT) {
      const int dd = c >> 3, kc = c & 7;
      const u32x4_t y = *reinterpret_cast<const u32x4_t *>(tile + ((size_t)k * 128 + dd) * kVtPitch + kc * 8);
      *reinterpret_cast<u32x4_t *>(vt + ((size_t)g[k] * D + dd) * vts + r0[k] + kc * 8) = y;
    }
}

// Lays the workspace out from `base` (nullptr: just measure), with `parts`
// split-K partial-tile slots for bf16 projections.
inline Workspace carve(const srp_dims &d, const srp_batch &b, char *base, int parts = kGemmParts) {
  const size_t T = (size_t)(b.total_rows > 0 ? b.total_rows : 1);
  const size_t nr = (size_t)b.n_req;
  const size_t es = d.dtype == SRP_BF16 ? 2 : 4;
  const size_t kvd = (size_t)d.n_kv_heads * d.head_dim, qd = (size_t)d.n_heads * d.head_dim;
  Workspace w{};
  size_t off = 0;
  auto take = [&](size_t n) -> char * {
    char *p = base ? base + off : nullptr;
    off = align_up(off + n, 256);
    return p;
  };
  w.row_delta = (int32_t *)take(T * 4);
  w.row_req = (int32_t *)take(T * 4);
  w.rowflag = (uint8_t *)take(T);
  w.rlist = (int32_t *)take(T * 4);
  w.roff = (int32_t *)take((nr + 1) * 4);
  {
    const size_t nb = nr * (size_t)blocks_per_req(b.max_req_rows) + 1;
    w.blkcnt = (int32_t *)take((nb > 2 * nr + 2 ? nb : 2 * nr + 2) * 4);
  }
  w.dev_part = (float *)take(T * 2 * d.n_kv_heads * 4);
  w.fresh_kv = take(T * 2 * kvd * es);
  w.keys = (uint32_t *)take(T * 4);
  w.eflag = (uint8_t *)take(T);
  w.seq_ent = (int32_t *)take(T * 4);
  w.seq_pre = (int32_t *)take(T * 4);
  w.seq_flag = (uint8_t *)take(T);
  w.tsel_row = (int32_t *)take(T * 4);
  w.tsel_ent = (int32_t *)take(T * 4);
  w.sel_cnt = (int32_t *)take(nr * 4);
  w.sel_ent = (int32_t *)take(T * 4);
  w.q = take(T * qd * es);
  w.vt = d.dtype == SRP_BF16 ? take((size_t)d.n_kv_heads * d.head_dim * vt_stride(b.total_rows) * 2) : nullptr;
  w.tiles = (int32_t *)take((size_t)3 * max_attn_tiles((int)T, (int)nr) * 4);
  w.ctr = (int32_t *)take(16 * 4);
  w.gemm_parts = d.dtype == SRP_BF16 ? parts : 0;
  w.gemm_part = w.gemm_parts > 0 ? (float *)take((size_t)w.gemm_parts * kGemmPartFloats * 4) : nullptr;
  if (b.block_rows > 0) {
    w.row_slot = (int32_t *)take(T * 4);
    w.k_lin = take(T * kvd * es);
    w.v_lin = d.dtype == SRP_BF16 ? nullptr : take(T * kvd * es);  // bf16 transposes V from the pool
  }
  w.bytes = off;
  return w;
}

}  // namespace srp
