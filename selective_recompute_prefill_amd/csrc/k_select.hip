// Token selection of one layer: row metadata, candidate lists, per-request top-k
// by KV deviation with sliding-window grouping, CSR compaction, and the scatter of
// the fresh K/V rows into the cache (gfx950).
//
// One work-group of 1024 threads owns a request during selection. Every pass walks
// the request's entries in tiles of 1024 consecutive entries, so each thread owns
// the same entry position in every pass and per-entry data it wrote earlier is its
// own. The k-th largest squared deviation is found by an MSB-first radix select on
// the fp32 bit patterns (order-preserving for non-negative floats); ties at the
// threshold are taken in row order, so the result is deterministic.
#include "kernels.hpp"

namespace srp {

// ------------------------------------------------------------------------- //
// row metadata
// ------------------------------------------------------------------------- //
__global__ void row_meta_kernel(SelectArgs a, Workspace w) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < a.T; j += gridDim.x * blockDim.x) {
    const int c = upper_index(a.chunk_offsets, a.n_chunks + 1, j);
    const int src0 = a.chunk_src_pos[c];
    w.row_delta[j] = src0 >= 0 ? a.positions[j] - (src0 + j - a.chunk_offsets[c]) : kFresh;
    w.row_req[j] = upper_index(a.req_offsets, a.n_req + 1, j);
    w.rowflag[j] = 0;
    if (a.dev_out) a.dev_out[j] = __int_as_float(0x7fc00000);
  }
}

__global__ void mark_cand_kernel(SelectArgs a, Workspace w) {
  const int n = a.cand_offsets[a.n_req];
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int row = a.cand[i];
    if (row >= 0 && row < a.T && w.row_delta[row] != kFresh) w.rowflag[row] = kCand;
  }
}

// R = candidate rows plus fresh rows, compacted per request (3 passes over blocks
// of 1024 rows: count, scan of the block counts, write).
__device__ __forceinline__ bool in_r(const Workspace &w, int j) {
  return w.rowflag[j] || w.row_delta[j] == kFresh;
}

__global__ __launch_bounds__(1024) void r_count_kernel(SelectArgs a, Workspace w, int bpr) {
  __shared__ int sh[17];
  const int r = blockIdx.x / bpr, b = blockIdx.x - r * bpr;
  const int j = a.req_offsets[r] + b * 1024 + threadIdx.x;
  const int v = j < a.req_offsets[r + 1] ? (int)in_r(w, j) : 0;
  const int tot = block_sum(v, sh);
  if (threadIdx.x == 0) w.blkcnt[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void r_scan_kernel(SelectArgs a, Workspace w, int bpr) {
  __shared__ int sh[17];
  const int n = a.n_req * bpr;
  int carry = 0;
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const int v = i < n ? w.blkcnt[i] : 0;
    int tot;
    const int p = block_excl_scan(v, sh, &tot) + carry;
    if (i < n) {
      w.blkcnt[i] = p;
      if (i % bpr == 0) w.roff[i / bpr] = p;
    }
    carry += tot;
  }
  if (threadIdx.x == 0) {
    w.roff[a.n_req] = carry;
    w.ctr[kCtrREntries] = carry;
  }
}

__global__ __launch_bounds__(1024) void r_write_kernel(SelectArgs a, Workspace w, int bpr) {
  __shared__ int sh[17];
  const int r = blockIdx.x / bpr, b = blockIdx.x - r * bpr;
  const int j = a.req_offsets[r] + b * 1024 + threadIdx.x;
  const int v = j < a.req_offsets[r + 1] ? (int)in_r(w, j) : 0;
  int tot;
  const int p = block_excl_scan(v, sh, &tot);
  if (v) w.rlist[w.blkcnt[blockIdx.x] + p] = j;
}

// ------------------------------------------------------------------------- //
// selection: one work-group per request
// ------------------------------------------------------------------------- //
__global__ __launch_bounds__(1024) void select_kernel(SelectArgs a, Workspace w) {
  __shared__ int sh[17];
  __shared__ int hist[256];
  __shared__ int digit_info[2];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int *roff = a.cand ? w.roff : a.req_offsets;
  const int e0 = roff[r], e1 = roff[r + 1];
  const int rq0 = a.req_offsets[r], rq1 = a.req_offsets[r + 1];
  const int P0 = a.dev_mode == SRP_DEV_V ? a.nkv : 0, P1 = 2 * a.nkv;

  // cached rows of the request (the N of the ratio)
  int my_ctx = 0;
  for (int j = rq0 + tid; j < rq1; j += 1024) my_ctx += w.row_delta[j] != kFresh;
  const int n_ctx = block_sum(my_ctx, sh);

  // entry flags and keys
  int my_cand = 0;
  for (int e = e0 + tid; e < e1; e += 1024) {
    const int row = a.cand ? w.rlist[e] : e;
    uint8_t fl;
    if (w.row_delta[row] == kFresh) {
      fl = kFreshF;
    } else {
      fl = kCand;
      float s = 0.f;
      const float *dp = w.dev_part + (size_t)e * 2 * a.nkv;
      for (int p = P0; p < P1; ++p) s += dp[p];
      w.keys[e] = __float_as_uint(s);
      if (a.dev_out) a.dev_out[row] = sqrtf(s);
      ++my_cand;
    }
    w.eflag[e] = fl;
  }
  const int n_cand = block_sum(my_cand, sh);

  int k;
  if (a.mode == SRP_SEL_GIVEN) {
    k = n_cand;
  } else {
    const double kd = floor(a.ratio * (double)n_ctx + 0.5);
    k = kd < (double)n_cand ? (int)kd : n_cand;
  }

  if (k >= n_cand) {
    for (int e = e0 + tid; e < e1; e += 1024)
      if (w.eflag[e] & kCand) w.eflag[e] |= kTop;
  } else if (k > 0) {
    uint32_t prefix = 0, pmask = 0;
    int need = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int e = e0 + tid; e < e1; e += 1024) {
        if (!(w.eflag[e] & kCand)) continue;
        const uint32_t key = w.keys[e];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns digits 255-4l .. 252-4l (descending); find the digit where
        // the count of keys at or above it first reaches `need`
        int c[4], s4 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { c[q] = hist[255 - 4 * tid - q]; s4 += c[q]; }
        const int incl = wave_incl_scan(s4);
        int above = incl - s4;
        const bool mine = above < need && incl >= need;
        if (mine) {
          int dsel = 0, abv = above;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (abv + c[q] >= need) { dsel = 255 - 4 * tid - q; break; }
            abv += c[q];
          }
          digit_info[0] = dsel;
          digit_info[1] = abv;
        }
      }
      __syncthreads();
      const uint32_t dsel = (uint32_t)digit_info[0];
      need -= digit_info[1];
      prefix |= dsel << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    // prefix = the k-th largest key; take every larger key and the first `need`
    // equal keys in entry (row) order
    int eq_run = 0;
    for (int base = e0; base < e1; base += 1024) {
      const int e = base + tid;
      bool gt = false, eq = false;
      if (e < e1 && (w.eflag[e] & kCand)) {
        const uint32_t key = w.keys[e];
        gt = key > prefix;
        eq = key == prefix;
      }
      int eq_tot;
      const int eqp = block_excl_scan(eq ? 1 : 0, sh, &eq_tot) + eq_run;
      if (gt || (eq && eqp < need)) w.eflag[e] |= kTop;
      eq_run += eq_tot;
    }
  }
  __threadfence_block();
  __syncthreads();

  if (a.window > 0) {
    // the grouping sequence: the request's candidate rows in order
    const int win = a.window;
    int carry = 0;
    for (int base = e0; base < e1; base += 1024) {
      const int e = base + tid;
      const uint8_t fl = e < e1 ? w.eflag[e] : 0;
      const int c = (fl & kCand) ? 1 : 0;
      int tot;
      const int slot = block_excl_scan(c, sh, &tot) + carry;
      if (c) {
        w.seq_ent[e0 + slot] = e;
        w.seq_flag[e0 + slot] = (fl & kTop) ? 1 : 0;
      }
      carry += tot;
    }
    const int n_seq = carry;
    __threadfence_block();
    __syncthreads();
    carry = 0;
    for (int base = 0; base < n_seq; base += 1024) {
      const int s = base + tid;
      const int v = s < n_seq ? (w.seq_flag[e0 + s] & 1) : 0;
      int tot;
      const int p = block_excl_scan(v, sh, &tot) + carry;
      if (s < n_seq) w.seq_pre[e0 + s] = p + v;  // inclusive count of top slots
      carry += tot;
    }
    __threadfence_block();
    __syncthreads();
    for (int t = tid; t < n_seq; t += 1024) {
      const uint8_t f = w.seq_flag[e0 + t];
      bool pass = false;
      if ((f & 1) && t + win <= n_seq) {
        const int cnt = w.seq_pre[e0 + t + win - 1] - (t > 0 ? w.seq_pre[e0 + t - 1] : 0);
        pass = cnt >= a.tau;
      }
      if (pass) w.seq_flag[e0 + t] = f | 2;
    }
    __threadfence_block();
    __syncthreads();
    for (int p = tid; p < n_seq; p += 1024) {
      bool kept = false;
      const int t0 = p - win + 1 > 0 ? p - win + 1 : 0;
      for (int t = t0; t <= p; ++t) kept |= (w.seq_flag[e0 + t] & 2) != 0;
      if (kept) {
        const int e = w.seq_ent[e0 + p];
        w.eflag[e] |= kSel;
      }
    }
    __threadfence_block();
    __syncthreads();
  }

  // compact the request's selection (fresh rows included) in row order
  const uint8_t want = a.window > 0 ? kSel : kTop;
  int carry = 0;
  for (int base = e0; base < e1; base += 1024) {
    const int e = base + tid;
    const uint8_t fl = e < e1 ? w.eflag[e] : 0;
    const int s = ((fl & kFreshF) || (fl & want)) ? 1 : 0;
    int tot;
    const int p = block_excl_scan(s, sh, &tot) + carry;
    if (s) {
      w.tsel_row[e0 + p] = a.cand ? w.rlist[e] : e;
      w.tsel_ent[e0 + p] = e;
    }
    carry += tot;
  }
  if (tid == 0) w.sel_cnt[r] = carry;
}

// ------------------------------------------------------------------------- //
// finalize: CSR offsets and the attention tile list (longest first)
// ------------------------------------------------------------------------- //
__global__ __launch_bounds__(1024) void finalize_kernel(SelectArgs a, Workspace w, int32_t *sel_offsets) {
  __shared__ int sh[17];
  const int nr = a.n_req, tid = threadIdx.x;
  int32_t *ntile = w.blkcnt;            // [nr] tiles per request
  int32_t *tpre = w.blkcnt + nr + 1;    // [nr+1] exclusive prefix of ntile
  int carry = 0, tcarry = 0;
  for (int base = 0; base < nr; base += 1024) {
    const int r = base + tid;
    const int c = r < nr ? w.sel_cnt[r] : 0;
    const int nt = (c + kQT - 1) / kQT;
    int tot, ttot;
    const int p = block_excl_scan(c, sh, &tot) + carry;
    const int tp = block_excl_scan(nt, sh, &ttot) + tcarry;
    if (r < nr) {
      sel_offsets[r] = p;
      ntile[r] = nt;
      tpre[r] = tp;
    }
    carry += tot;
    tcarry += ttot;
  }
  if (tid == 0) {
    sel_offsets[nr] = carry;
    tpre[nr] = tcarry;
    w.ctr[kCtrTotalSel] = carry;
    w.ctr[kCtrTiles] = tcarry;
  }
  __threadfence_block();
  __syncthreads();
  // tile i of request r is emitted at E = (tiles of any request with index > i)
  // + (requests before r that also have a tile i): descending tile index first,
  // so the longest causal ranges start first.
  for (int f = tid; f < tcarry; f += 1024) {
    const int r = upper_index(tpre, nr + 1, f);
    const int i = f - tpre[r];
    int E = 0;
    for (int q = 0; q < nr; ++q) {
      const int t = ntile[q];
      E += t - 1 - i > 0 ? t - 1 - i : 0;
      if (q < r && t > i) ++E;
    }
    const int c = w.sel_cnt[r];
    w.tiles[3 * E + 0] = sel_offsets[r] + i * kQT;
    w.tiles[3 * E + 1] = c - i * kQT < kQT ? c - i * kQT : kQT;
    w.tiles[3 * E + 2] = r;
  }
}

// ------------------------------------------------------------------------- //
// compaction to sel_idx and scatter of the fresh K/V rows (one wave per entry)
// ------------------------------------------------------------------------- //
template <typename T>
__global__ __launch_bounds__(256) void compact_scatter_kernel(SelectArgs a, Workspace w, int kvdim,
                                                              int32_t *sel_idx, const int32_t *sel_offsets,
                                                              T *k_cache, T *v_cache) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int *roff = a.cand ? w.roff : a.req_offsets;
  const int nR = roff[a.n_req];
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte chunk
  const int chunks = kvdim / V;
  for (int q = wave; q < nR; q += nwaves) {
    const int r = upper_index(roff, a.n_req + 1, q);
    const int i = q - roff[r];
    if (i >= w.sel_cnt[r]) continue;
    const int out = sel_offsets[r] + i;
    const int row = w.tsel_row[q];
    const int e = w.tsel_ent[q];
    if (lane == 0) {
      sel_idx[out] = row;
      w.sel_ent[out] = e;
    }
    const T *f = (const T *)w.fresh_kv + (size_t)e * 2 * kvdim;
    for (int c = lane; c < chunks; c += 64) {
      *reinterpret_cast<uint4 *>(k_cache + (size_t)row * kvdim + c * V) =
          *reinterpret_cast<const uint4 *>(f + c * V);
      *reinterpret_cast<uint4 *>(v_cache + (size_t)row * kvdim + c * V) =
          *reinterpret_cast<const uint4 *>(f + kvdim + c * V);
    }
  }
}

// ------------------------------------------------------------------------- //
// launchers
// ------------------------------------------------------------------------- //
hipError_t launch_prepare(const SelectArgs &a, const Workspace &w, hipStream_t s) {
  if (a.T > 0) {
    int grid = (a.T + 255) / 256;
    grid = grid < 4096 ? grid : 4096;
    hipLaunchKernelGGL(row_meta_kernel, dim3(grid), dim3(256), 0, s, a, w);
  }
  if (a.cand) {
    int grid = (a.T + 255) / 256;
    grid = grid < 1024 ? (grid > 0 ? grid : 1) : 1024;
    hipLaunchKernelGGL(mark_cand_kernel, dim3(grid), dim3(256), 0, s, a, w);
    const int bpr = blocks_per_req(a.max_req_rows);
    hipLaunchKernelGGL(r_count_kernel, dim3(a.n_req * bpr), dim3(1024), 0, s, a, w, bpr);
    hipLaunchKernelGGL(r_scan_kernel, dim3(1), dim3(1024), 0, s, a, w, bpr);
    hipLaunchKernelGGL(r_write_kernel, dim3(a.n_req * bpr), dim3(1024), 0, s, a, w, bpr);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs &a, const Workspace &w, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(a.n_req), dim3(1024), 0, s, a, w);
  return hipGetLastError();
}

hipError_t launch_finalize(const SelectArgs &a, const Workspace &w, int32_t *sel_offsets, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, s, a, w, sel_offsets);
  return hipGetLastError();
}

hipError_t launch_compact_scatter(const SelectArgs &a, const Workspace &w, int dtype, int kvdim,
                                  int32_t *sel_idx, const int32_t *sel_offsets, void *k_cache,
                                  void *v_cache, hipStream_t s) {
  int grid = (a.T * 64 + 255) / 256;
  grid = grid < 2048 ? (grid > 0 ? grid : 1) : 2048;
  if (dtype == SRP_BF16)
    hipLaunchKernelGGL(compact_scatter_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, a, w, kvdim,
                       sel_idx, sel_offsets, (uint16_t *)k_cache, (uint16_t *)v_cache);
  else
    hipLaunchKernelGGL(compact_scatter_kernel<float>, dim3(grid), dim3(256), 0, s, a, w, kvdim,
                       sel_idx, sel_offsets, (float *)k_cache, (float *)v_cache);
  return hipGetLastError();
}

}  // namespace srp
