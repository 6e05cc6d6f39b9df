// Token selection of one layer: row metadata, candidate lists, per-request top-k
// by KV deviation with sliding-window grouping, CSR compaction, and the scatter of
// the fresh K/V rows into the cache (gfx950).
//
// Squared deviations are summed grid-wide; then one work-group of 1024 threads owns
// a request: order-free passes (counts, histograms, marks) stride over its entries
// so loads coalesce, and order-dependent scans run over pages of entry flags
// staged in LDS, each thread walking a contiguous segment. The k-th largest squared deviation is found by an MSB-first
// radix select on the fp32 bit patterns (order-preserving for non-negative floats);
// ties at the threshold are taken in row order, so the result is deterministic.
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
// keys: squared deviation of every candidate entry (grid-wide, fixed-order sum of
// the per-head partials), entry flags, and the optional deviation output
// ------------------------------------------------------------------------- //
__global__ __launch_bounds__(256) void keys_kernel(SelectArgs a, Workspace w) {
  const int *roff = a.cand ? w.roff : a.req_offsets;
  const int nR = roff[a.n_req];
  const int P0 = a.dev_mode == SRP_DEV_V ? a.nkv : 0, P1 = 2 * a.nkv;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < nR; e += gridDim.x * blockDim.x) {
    const int row = a.cand ? w.rlist[e] : e;
    if (w.row_delta[row] == kFresh) {
      w.eflag[e] = kFreshF;
      continue;
    }
    const float *dp = w.dev_part + (size_t)e * 2 * a.nkv;
    float s = 0.f;
    for (int p = P0; p < P1; ++p) s += dp[p];
    w.keys[e] = __float_as_uint(s);
    w.eflag[e] = kCand;
    if (a.dev_out) a.dev_out[row] = sqrtf(s);
  }
}

// ------------------------------------------------------------------------- //
// selection: one work-group per request
// ------------------------------------------------------------------------- //
// [lo, hi): the contiguous share of n items owned by this thread
__device__ __forceinline__ void my_segment(int n, int &lo, int &hi) {
  const int per = (n + (int)blockDim.x - 1) / (int)blockDim.x;
  lo = min(n, (int)threadIdx.x * per);
  hi = min(n, lo + per);
}

constexpr int kHistBins = 4096;
constexpr int kPage = 32768;  // entries whose flags are staged in LDS at a time

__global__ __launch_bounds__(1024) void select_kernel(SelectArgs a, Workspace w) {
  __shared__ int sh[17];
  __shared__ int hist[kHistBins];
  __shared__ int digit_info[2];
  __shared__ uint8_t pg[kPage];
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int *roff = a.cand ? w.roff : a.req_offsets;
  const int e0 = roff[r], e1 = roff[r + 1];
  const int rq0 = a.req_offsets[r], rq1 = a.req_offsets[r + 1];

  // cached rows of the request (the N of the ratio) and its candidates; loops
  // whose result does not depend on order stride over the entries (coalesced)
  int my_ctx = 0, my_cand = 0;
  for (int j = rq0 + tid; j < rq1; j += nt) my_ctx += w.row_delta[j] != kFresh;
  for (int e = e0 + tid; e < e1; e += nt) my_cand += (w.eflag[e] & kCand) ? 1 : 0;
  const int n_ctx = block_sum(my_ctx, sh);
  const int n_cand = block_sum(my_cand, sh);

  int k;
  if (a.mode == SRP_SEL_GIVEN) {
    k = n_cand;
  } else {
    const double kd = floor(a.ratio * (double)n_ctx + 0.5);
    k = kd < (double)n_cand ? (int)kd : n_cand;
  }

  if (k >= n_cand) {
    for (int e = e0 + tid; e < e1; e += nt)
      if (w.eflag[e] & kCand) w.eflag[e] |= kTop;
  } else if (k > 0) {
    // radix select of the k-th largest key, digits of 12, 12 and 8 bits from
    // the top (the first pass splits sign, exponent and 3 mantissa bits)
    uint32_t prefix = 0, pmask = 0;
    int need = k;
    const int shifts[3] = {20, 8, 0}, widths[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = shifts[pass], nb = 1 << widths[pass];
      const uint32_t dmask = (uint32_t)nb - 1u;
      for (int b = tid; b < nb; b += nt) hist[b] = 0;
      __syncthreads();
      for (int e = e0 + tid; e < e1; e += nt) {
        if (!(w.eflag[e] & kCand)) continue;
        const uint32_t key = w.keys[e];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1);
      }
      __syncthreads();
      // thread t owns 4 digits in descending order: nb-1-4t .. nb-4-4t
      int c[4], s4 = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dg = nb - 1 - 4 * tid - q;
        c[q] = dg >= 0 ? hist[dg] : 0;
        s4 += c[q];
      }
      int tot;
      const int above = block_excl_scan(s4, sh, &tot);
      if (above < need && above + s4 >= need) {
        int abv = above, dsel = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (abv + c[q] >= need) { dsel = nb - 1 - 4 * tid - q; break; }
          abv += c[q];
        }
        digit_info[0] = dsel;
        digit_info[1] = abv;
      }
      __syncthreads();
      need -= digit_info[1];
      prefix |= (uint32_t)digit_info[0] << shift;
      pmask |= dmask << shift;
      __syncthreads();
    }
    // prefix = the k-th largest key: take every larger key and the first `need`
    // keys equal to it in entry (row) order
    int my_eq = 0;
    for (int e = e0 + tid; e < e1; e += nt) {
      if (!(w.eflag[e] & kCand)) continue;
      const uint32_t key = w.keys[e];
      if (key > prefix) w.eflag[e] |= kTop;
      else if (key == prefix) ++my_eq;
    }
    const int eq_tot = block_sum(my_eq, sh);
    if (eq_tot == need) {
      for (int e = e0 + tid; e < e1; e += nt)
        if ((w.eflag[e] & kCand) && w.keys[e] == prefix) w.eflag[e] |= kTop;
    } else {
      // several equal keys at the threshold: rank them in row order
      int eq_run = 0;
      for (int base = e0; base < e1; base += nt) {
        const int e = base + tid;
        const bool eq = e < e1 && (w.eflag[e] & kCand) && w.keys[e] == prefix;
        int t;
        const int rank = block_excl_scan(eq ? 1 : 0, sh, &t) + eq_run;
        if (eq && rank < need) w.eflag[e] |= kTop;
        eq_run += t;
      }
    }
  }
  __threadfence_block();
  __syncthreads();

  if (a.window > 0) {
    // the grouping sequence: the request's candidate rows in order; slot numbers
    // and the inclusive count of top-k slots come from one ordered walk over pages
    // of entry flags staged in LDS
    const int win = a.window;
    int carry_c = 0, carry_t = 0;
    for (int pb = e0; pb < e1; pb += kPage) {
      const int np = min(kPage, e1 - pb);
      for (int i = tid; i < np; i += nt) pg[i] = w.eflag[pb + i];
      __syncthreads();
      int lo, hi;
      my_segment(np, lo, hi);
      int c = 0, t = 0;
      for (int i = lo; i < hi; ++i) {
        const uint8_t fl = pg[i];
        if (fl & kCand) { ++c; t += (fl & kTop) ? 1 : 0; }
      }
      int ctot, ttot;
      int cb = block_excl_scan(c, sh, &ctot);
      int tb = block_excl_scan(t, sh, &ttot);
      for (int i = lo; i < hi; ++i) {
        const uint8_t fl = pg[i];
        if (!(fl & kCand)) continue;
        const int top = (fl & kTop) ? 1 : 0;
        const int slot = carry_c + cb++;
        tb += top;
        w.seq_ent[e0 + slot] = pb + i;
        w.seq_flag[e0 + slot] = (uint8_t)top;
        w.seq_pre[e0 + slot] = carry_t + tb;
      }
      carry_c += ctot;
      carry_t += ttot;
      __syncthreads();
    }
    const int n_seq = carry_c;
    __threadfence_block();
    __syncthreads();
    for (int t = tid; t < n_seq; t += nt) {
      const uint8_t f = w.seq_flag[e0 + t];
      if ((f & 1) && t + win <= n_seq) {
        const int cnt = w.seq_pre[e0 + t + win - 1] - (t > 0 ? w.seq_pre[e0 + t - 1] : 0);
        if (cnt >= a.tau) w.seq_flag[e0 + t] = f | 2;
      }
    }
    __threadfence_block();
    __syncthreads();
    for (int p = tid; p < n_seq; p += nt) {
      bool kept = false;
      const int t0 = p - win + 1 > 0 ? p - win + 1 : 0;
      for (int t = t0; t <= p; ++t) kept |= (w.seq_flag[e0 + t] & 2) != 0;
      if (kept) w.eflag[w.seq_ent[e0 + p]] |= kSel;
    }
    __threadfence_block();
    __syncthreads();
  }

  // compact the request's selection (fresh rows included) in row order
  const uint8_t want = a.window > 0 ? kSel : kTop;
  int carry = 0;
  for (int pb = e0; pb < e1; pb += kPage) {
    const int np = min(kPage, e1 - pb);
    for (int i = tid; i < np; i += nt) pg[i] = w.eflag[pb + i];
    __syncthreads();
    int lo, hi;
    my_segment(np, lo, hi);
    int c = 0;
    for (int i = lo; i < hi; ++i) c += ((pg[i] & kFreshF) || (pg[i] & want)) ? 1 : 0;
    int tot;
    int p = block_excl_scan(c, sh, &tot) + carry;
    for (int i = lo; i < hi; ++i) {
      if ((pg[i] & kFreshF) || (pg[i] & want)) {
        const int e = pb + i;
        w.tsel_row[e0 + p] = a.cand ? w.rlist[e] : e;
        w.tsel_ent[e0 + p] = e;
        ++p;
      }
    }
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) w.sel_cnt[r] = carry;
}

// ------------------------------------------------------------------------- //
// selection with the request resident in LDS (requests of up to kLdsEntries
// entries): keys and flags are loaded once; after marking, the key storage holds
// the grouping sequence as 16-bit entry offsets and prefix counts
// ------------------------------------------------------------------------- //
constexpr int kLdsEntries = 22528;

__device__ __forceinline__ int radix_digit_pass(const uint32_t *keys, const uint8_t *fl, int n,
                                                uint32_t prefix, uint32_t pmask, int shift, int nb,
                                                int need, int *hist, int *sh, int *digit_info,
                                                int *above_out) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const uint32_t dmask = (uint32_t)nb - 1u;
  for (int b = tid; b < nb; b += nt) hist[b] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += nt) {
    if (!(fl[i] & kCand)) continue;
    const uint32_t key = keys[i];
    if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1);
  }
  __syncthreads();
  int c[4], s4 = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int dg = nb - 1 - 4 * tid - q;
    c[q] = dg >= 0 ? hist[dg] : 0;
    s4 += c[q];
  }
  int tot;
  const int above = block_excl_scan(s4, sh, &tot);
  if (above < need && above + s4 >= need) {
    int abv = above, dsel = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (abv + c[q] >= need) { dsel = nb - 1 - 4 * tid - q; break; }
      abv += c[q];
    }
    digit_info[0] = dsel;
    digit_info[1] = abv;
  }
  __syncthreads();
  *above_out = digit_info[1];
  const int d = digit_info[0];
  __syncthreads();
  return d;
}

__global__ __launch_bounds__(1024) void select_lds_kernel(SelectArgs a, Workspace w) {
  __shared__ int sh[17];
  __shared__ int hist[kHistBins];
  __shared__ int digit_info[2];
  __shared__ uint32_t keys_s[kLdsEntries];  // later: seq_ent (u16) | seq_pre (u16)
  __shared__ uint8_t fl_s[kLdsEntries];
  __shared__ uint8_t sq_s[kLdsEntries];      // grouping: bit 0 top-k slot, bit 1 passing window
  __shared__ int sh_max[1024];               // grouping: max-scan of passing starts
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int *roff = a.cand ? w.roff : a.req_offsets;
  const int e0 = roff[r], e1 = roff[r + 1], n = e1 - e0;

  int my_cand = 0;
  for (int i = tid; i < n; i += 4 * nt) {
    // four independent loads of flags and keys per thread before any store
    uint8_t f[4];
    uint32_t k4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = i + u * nt;
      f[u] = j < n ? w.eflag[e0 + j] : 0;
      k4[u] = j < n ? w.keys[e0 + j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = i + u * nt;
      if (j < n) {
        fl_s[j] = f[u];
        keys_s[j] = (f[u] & kCand) ? k4[u] : 0u;
        my_cand += (f[u] & kCand) ? 1 : 0;
      }
    }
  }
  int my_ctx = 0;
  if (a.cand) {
    for (int j = a.req_offsets[r] + tid; j < a.req_offsets[r + 1]; j += nt) my_ctx += w.row_delta[j] != kFresh;
  } else {
    my_ctx = my_cand;  // every cached row of the request is a candidate
  }
  const int n_cand = block_sum(my_cand, sh);
  const int n_ctx = block_sum(my_ctx, sh);

  int k;
  if (a.mode == SRP_SEL_GIVEN) {
    k = n_cand;
  } else {
    const double kd = floor(a.ratio * (double)n_ctx + 0.5);
    k = kd < (double)n_cand ? (int)kd : n_cand;
  }
  if (k >= n_cand) {
    for (int i = tid; i < n; i += nt)
      if (fl_s[i] & kCand) fl_s[i] |= kTop;
  } else if (k > 0) {
    uint32_t prefix = 0, pmask = 0;
    int need = k;
    const int shifts[3] = {20, 8, 0}, widths[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
      int above;
      const int d = radix_digit_pass(keys_s, fl_s, n, prefix, pmask, shifts[pass], 1 << widths[pass],
                                     need, hist, sh, digit_info, &above);
      need -= above;
      prefix |= (uint32_t)d << shifts[pass];
      pmask |= ((1u << widths[pass]) - 1u) << shifts[pass];
    }
    int my_eq = 0;
    for (int i = tid; i < n; i += nt) {
      if (!(fl_s[i] & kCand)) continue;
      if (keys_s[i] > prefix) fl_s[i] |= kTop;
      else if (keys_s[i] == prefix) ++my_eq;
    }
    const int eq_tot = block_sum(my_eq, sh);
    if (eq_tot == need) {
      for (int i = tid; i < n; i += nt)
        if ((fl_s[i] & kCand) && keys_s[i] == prefix) fl_s[i] |= kTop;
    } else {
      // several equal keys at the threshold: the first `need` in row order
      int lo, hi;
      my_segment(n, lo, hi);
      int c = 0;
      for (int i = lo; i < hi; ++i) c += ((fl_s[i] & kCand) && keys_s[i] == prefix) ? 1 : 0;
      int t;
      int rank = block_excl_scan(c, sh, &t);
      for (int i = lo; i < hi; ++i)
        if ((fl_s[i] & kCand) && keys_s[i] == prefix) {
          if (rank < need) fl_s[i] |= kTop;
          ++rank;
        }
    }
  }
  __syncthreads();

  if (a.window > 0) {
    const int win = a.window;
    uint16_t *seq_ent = reinterpret_cast<uint16_t *>(keys_s);   // [n] slot -> entry offset
    uint16_t *seq_pre = seq_ent + kLdsEntries;                  // [n] inclusive top count
    int lo, hi;
    my_segment(n, lo, hi);
    int c = 0, tp = 0;
    for (int i = lo; i < hi; ++i)
      if (fl_s[i] & kCand) { ++c; tp += (fl_s[i] & kTop) ? 1 : 0; }
    int n_seq, n_top;
    int slot = block_excl_scan(c, sh, &n_seq);
    int run = block_excl_scan(tp, sh, &n_top);
    for (int i = lo; i < hi; ++i) {
      const uint8_t f = fl_s[i];
      if (!(f & kCand)) continue;
      const int top = (f & kTop) ? 1 : 0;
      run += top;
      seq_ent[slot] = (uint16_t)i;
      seq_pre[slot] = (uint16_t)run;
      sq_s[slot] = (uint8_t)top;
      ++slot;
    }
    __syncthreads();
    for (int t = tid; t < n_seq; t += nt) {
      if ((sq_s[t] & 1) && t + win <= n_seq) {
        const int cnt = (int)seq_pre[t + win - 1] - (t > 0 ? (int)seq_pre[t - 1] : 0);
        if (cnt >= a.tau) sq_s[t] |= 2;
      }
    }
    __syncthreads();
    // a slot is kept when the latest passing window start at or before it lies
    // within the window: a max-scan of passing starts over contiguous segments
    {
      int lo2, hi2;
      my_segment(n_seq, lo2, hi2);
      int last = -1;
      for (int t = lo2; t < hi2; ++t) last = (sq_s[t] & 2) ? t : last;
      // latest passing start before this segment: max over earlier segments
      sh_max[tid] = last;
      __syncthreads();
      for (int o = 1; o < nt; o <<= 1) {
        const int v = tid >= o ? sh_max[tid - o] : -1;
        __syncthreads();
        if (v > sh_max[tid]) sh_max[tid] = v;
        __syncthreads();
      }
      int run = tid > 0 ? sh_max[tid - 1] : -1;
      for (int t = lo2; t < hi2; ++t) {
        if (sq_s[t] & 2) run = t;
        if (run >= 0 && run > t - win) fl_s[seq_ent[t]] |= kSel;
      }
    }
    __syncthreads();
  }

  // compact the request's selection (fresh rows included) in row order
  const uint8_t want = a.window > 0 ? kSel : kTop;
  int lo, hi;
  my_segment(n, lo, hi);
  int c = 0;
  for (int i = lo; i < hi; ++i) c += ((fl_s[i] & kFreshF) || (fl_s[i] & want)) ? 1 : 0;
  int total;
  int p = block_excl_scan(c, sh, &total);
  for (int i = lo; i < hi; ++i) {
    if ((fl_s[i] & kFreshF) || (fl_s[i] & want)) {
      const int e = e0 + i;
      w.tsel_row[e0 + p] = a.cand ? w.rlist[e] : e;
      w.tsel_ent[e0 + p] = e;
      ++p;
    }
  }
  if (tid == 0) w.sel_cnt[r] = total;
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
    const int nt = (c + a.tile_rows - 1) / a.tile_rows;
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
    const int tr = a.tile_rows;
    w.tiles[3 * E + 0] = sel_offsets[r] + i * tr;
    w.tiles[3 * E + 1] = c - i * tr < tr ? c - i * tr : tr;
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
  int grid = (a.T + 255) / 256;
  grid = grid < 2048 ? (grid > 0 ? grid : 1) : 2048;
  hipLaunchKernelGGL(keys_kernel, dim3(grid), dim3(256), 0, s, a, w);
  if (a.max_req_rows <= kLdsEntries) {
    hipLaunchKernelGGL(select_lds_kernel, dim3(a.n_req), dim3(1024), 0, s, a, w);
    return hipGetLastError();
  }
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
