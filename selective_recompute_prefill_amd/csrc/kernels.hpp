// Host-side launchers of libsrp's kernels (internal to the library).
#pragma once

#include "common.hpp"

namespace srp {

enum EpiMode { EPI_KV = 0, EPI_Q = 1, EPI_ENC = 2, EPI_V = 3, EPI_QK = 4 };

// C[m, n] = sum_k A[row(m), k] * B[n, k], followed by an epilogue on each
// head-sized unit of a row:
//  EPI_KV : n < kvdim are K heads (roped at the row's global position), the rest
//           V heads. Fresh K/V go to `fresh` [m][2 kvdim]. For cached rows the
//           cached K is rotated by the row's delta (written back in place) and the
//           squared deviation of each head goes to dev_part [m][2 nkv].
//  EPI_Q  : n are Q heads, roped and multiplied by q_scale; written to q_out [m][qdim].
//  EPI_ENC: like EPI_KV's layout, K roped at positions[m]; K -> k_cache[m],
//           V -> v_cache[m].
//  EPI_V  : n are V heads only: fresh V to the V half of `fresh`, squared
//           deviation from the cached V to dev_part (V-only deviation).
//  EPI_QK : n < qdim are Q heads (as EPI_Q), the rest K heads, roped at the
//           row's position and written to the row's cache row in k_cache.
struct GemmArgs {
  int dtype;
  const void *A;       // [*, K]
  int K;
  const int32_t *a_rows;  // m -> row of A (NULL: identity)
  int M_host;
  const int32_t *M_dev;   // device M (overrides M_host when set)
  int M_cap;              // upper bound of M (grid sizing)
  const void *B;       // [N, K]
  int N;
  int mode;
  int nh, nkv, d;
  const int32_t *positions;
  const int32_t *row_delta;
  RopeTable rope;
  void *k_cache, *v_cache;
  void *fresh;
  float *dev_part;
  void *q_out;
  float q_scale;  // EPI_Q: factor applied to the roped queries
  const int32_t *row_slot;  // EPI_KV: cache row of each token row (paged cache), or NULL
  float *part;    // bf16: fp32 partial tiles of split tail tiles (kGemmPartFloats each), or NULL
  int part_cap;   // partial-tile slots at `part`
  int grid_main;  // set by launch_gemm: work-groups of the main kernel
  // EPI_Q / EPI_QK (bf16): the transposed V copy for the attention, built by
  // work-groups with no tile left (chunks claimed through vt_ctr, which must be
  // zero at launch); vt_dst NULL: none
  const void *vt_src;        // fused V cache
  const int32_t *vt_slot;    // cache row of each batch row (paged), or NULL
  void *vt_dst;              // [nkv][d][vt_stride]
  int vt_T, vt_stride;
  int32_t *vt_ctr;
};
hipError_t launch_gemm(const GemmArgs &g, hipStream_t s);

// Rows of one request that the LDS-resident selection kernels hold (larger
// requests take the global-memory path; external-score selection needs this bound).
constexpr int kLdsEntries = 22528;

struct SelectArgs {
  int n_req, T, max_req_rows;
  const int32_t *req_offsets, *chunk_offsets, *chunk_src_pos, *positions;
  int n_chunks;
  int mode, window, tau, dev_mode;
  double ratio;
  const int32_t *cand, *cand_offsets;
  int nkv;
  float *dev_out;
  int tile_rows;  // selected rows per attention tile
  int k_ceil;     // k = ceil(ratio * N) instead of round half up
  bool listed;    // the recomputed rows are an explicit per-request list (R list)
  // external scores and span completion (SRP_SEL_SCORES)
  const float *scores;
  int span_max;
  double tau_smooth, tau_cover, cap_ratio;
  int fresh_all;  // scatter fresh K/V of every recomputed row
  bool v_only;    // V-only fast path: only fresh V is scattered (K comes with Q)
  // paged cache (block_rows > 0): pool row of segment c's row i =
  // block_table[seg_block[c] + i / block_rows] * block_rows + i % block_rows
  int block_rows;
  const int32_t *seg_block, *block_table;
};
// Row metadata (delta, request), dev_out prefill with NaN, candidate marking, the
// score-based choice of rows in SRP_SEL_SCORES, and the R list (candidate or
// chosen rows plus fresh rows, per request) when the rows are listed.
hipError_t launch_prepare(const SelectArgs &a, const Workspace &w, hipStream_t s);
// Keys, top-k / grouping per request, then the CSR offsets and attention tiles.
hipError_t launch_select(const SelectArgs &a, const Workspace &w, int32_t *sel_offsets,
                         hipStream_t s);
hipError_t launch_compact_scatter(const SelectArgs &a, const Workspace &w, int dtype, int kvdim,
                                  int32_t *sel_idx, const int32_t *sel_offsets, void *k_cache,
                                  void *v_cache, hipStream_t s);
// Pool rows of a paged cache (block_rows = 0: row j is cache row j).
struct PagedMap {
  int block_rows;
  const int32_t *seg_block, *block_table;
};
__device__ __forceinline__ int paged_row(const PagedMap &pm, int c, int i) {
  return pm.block_table[pm.seg_block[c] + i / pm.block_rows] * pm.block_rows + i % pm.block_rows;
}

// Re-rotation of cached rows; with `skip` (row flags) rows flagged as candidates
// are left alone (the projection epilogue rotates those). row_delta and row_slot
// (optional): the rotation index (kFresh: none) and cache row of each row, else
// derived from the layout and `pm`.
hipError_t launch_rerotate(int dtype, int T, int nkv, int d, const int32_t *row_delta,
                           const int32_t *row_slot, const PagedMap &pm,
                           const int32_t *chunk_offsets, int n_chunks,
                           const int32_t *chunk_src_pos, const int32_t *positions,
                           const uint8_t *skip, const RopeTable &rt, void *k_cache, hipStream_t s);
// Paged cache: dst[j] = src[row_slot[j]] for the T rows of row_bytes each.
hipError_t launch_gather_rows(int T, size_t row_bytes, const int32_t *row_slot, const void *src,
                              void *dst, hipStream_t s);

struct AttnArgs {
  int dtype;
  int nh, nkv, d;
  const void *q;           // [n_sel][nh][d]; bf16: pre-multiplied by log2(e)/sqrt(d)
  const int32_t *sel_idx;  // [n_sel]
  const int32_t *req_offsets;
  const int32_t *tiles;    // [3 * max_tiles]: first selected row, count, request
  const int32_t *n_tiles;  // device
  int max_tiles;
  const void *k_cache, *v_cache;
  const void *vt;          // bf16: V transposed, [nkv][d][vt_stride]
  int vt_stride;
  int total_rows;
  void *out;               // [n_sel][nh][d]
};
hipError_t launch_attention(const AttnArgs &a, hipStream_t s);
// Selected rows per attention tile for this shape: bf16 packs (query, head)
// pairs of a KV group into 256 columns, floor(256 / G) queries for G = nh / nkv
// <= 8 (so at least 32); fp32 takes 32.
int attn_tile_rows(int dtype, int nh, int nkv);

hipError_t launch_residual_rmsnorm(int dtype, int H, void *hidden, const void *attn,
                                   const int32_t *sel_idx, const int32_t *total_dev,
                                   int cap, float eps, hipStream_t s);

}  // namespace srp
