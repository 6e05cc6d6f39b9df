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
__device__ __forceinline__ void row_meta(const SelectArgs &a, const Workspace &w, int j) {
  const int c = upper_index(a.chunk_offsets, a.n_chunks + 1, j);
  const int src0 = a.chunk_src_pos[c];
  w.row_delta[j] = src0 >= 0 ? a.positions[j] - (src0 + j - a.chunk_offsets[c]) : kFresh;
  w.row_req[j] = upper_index(a.req_offsets, a.n_req + 1, j);
  if (a.block_rows > 0)
    w.row_slot[j] = paged_row(PagedMap{a.block_rows, a.seg_block, a.block_table}, c, j - a.chunk_offsets[c]);
  w.rowflag[j] = 0;
  if (a.dev_out) a.dev_out[j] = __int_as_float(0x7fc00000);
}

__global__ void row_meta_kernel(SelectArgs a, Workspace w) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < a.T; j += gridDim.x * blockDim.x) row_meta(a, w, j);
}

__device__ __forceinline__ void mark_cand(const SelectArgs &a, const Workspace &w, int i) {
  const int row = a.cand[i];
  if (row >= 0 && row < a.T && w.row_delta[row] != kFresh) w.rowflag[row] = kCand;
}

__global__ void mark_cand_kernel(SelectArgs a, Workspace w) {
  const int n = a.cand_offsets[a.n_req];
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) mark_cand(a, w, i);
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

// The same three steps (row metadata, candidate marks, R list) in one work-group
// of 1024 threads, for batches of at most kPrepOneGroup rows: one launch instead of
// five, each of which costs more in launch and drain than in work at these sizes.
constexpr int kPrepOneGroup = 16384;
__global__ __launch_bounds__(1024) void prepare_one_group_kernel(SelectArgs a, Workspace w) {
  __shared__ int sh[17];
  const int tid = threadIdx.x;
  for (int j = tid; j < a.T; j += 1024) row_meta(a, w, j);
  __threadfence_block();
  __syncthreads();
  const int n = a.cand_offsets[a.n_req];
  for (int i = tid; i < n; i += 1024) mark_cand(a, w, i);
  __threadfence_block();
  __syncthreads();
  int carry = 0;
  for (int r = 0; r < a.n_req; ++r) {
    if (tid == 0) w.roff[r] = carry;
    const int end = a.req_offsets[r + 1];
    for (int base = a.req_offsets[r]; base < end; base += 1024) {
      const int j = base + tid;
      const int v = j < end ? (int)in_r(w, j) : 0;
      int tot;
      const int p = block_excl_scan(v, sh, &tot);
      if (v) w.rlist[carry + p] = j;
      carry += tot;
    }
  }
  if (tid == 0) {
    w.roff[a.n_req] = carry;
    w.ctr[kCtrREntries] = carry;
  }
}

// ------------------------------------------------------------------------- //
// keys: squared deviation of every candidate entry (grid-wide, fixed-order sum of
// the per-head partials), entry flags, and the optional deviation output
// ------------------------------------------------------------------------- //
__global__ __launch_bounds__(256) void keys_kernel(SelectArgs a, Workspace w) {
  const int *roff = a.listed ? w.roff : a.req_offsets;
  const int nR = roff[a.n_req];
  const int P0 = a.dev_mode == SRP_DEV_V ? a.nkv : 0, P1 = 2 * a.nkv;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < nR; e += gridDim.x * blockDim.x) {
    const int row = a.listed ? w.rlist[e] : e;
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

// k from the ratio: round half up, or ceil; the product is rounded on its own (no
// fused multiply-add), as a plain double evaluation of the formula does.
__device__ __forceinline__ int k_from_ratio(double ratio, int n_ctx, int n_cand, int k_ceil) {
#pragma clang fp contract(off)
  const double x = ratio * (double)n_ctx;
  const double kd = k_ceil ? ceil(x) : floor(x + 0.5);
  return kd < (double)n_cand ? (int)kd : n_cand;
}

__global__ __launch_bounds__(1024) void select_kernel(SelectArgs a, Workspace w) {
  __shared__ int sh[17];
  __shared__ int hist[kHistBins];
  __shared__ int digit_info[2];
  __shared__ uint8_t pg[kPage];
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int *roff = a.listed ? w.roff : a.req_offsets;
  const int e0 = roff[r], e1 = roff[r + 1];
  const int rq0 = a.req_offsets[r], rq1 = a.req_offsets[r + 1];

  // cached rows of the request (the N of the ratio) and its candidates; loops
  // whose result does not depend on order stride over the entries (coalesced)
  int my_ctx = 0, my_cand = 0;
  for (int j = rq0 + tid; j < rq1; j += nt) my_ctx += w.row_delta[j] != kFresh;
  for (int e = e0 + tid; e < e1; e += nt) my_cand += (w.eflag[e] & kCand) ? 1 : 0;
  const int n_ctx = block_sum(my_ctx, sh);
  const int n_cand = block_sum(my_cand, sh);

  const int k = a.mode == SRP_SEL_GIVEN ? n_cand : k_from_ratio(a.ratio, n_ctx, n_cand, a.k_ceil);

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
        w.tsel_row[e0 + p] = a.listed ? w.rlist[e] : e;
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
// finalize: CSR offsets and the attention tile list (longest first)
// ------------------------------------------------------------------------- //
// CSR offsets and the attention tile list of the whole batch (one work-group of
// 1024 threads, after every request's sel_cnt is written).
__device__ void finalize_body(const SelectArgs &a, const Workspace &w, int32_t *sel_offsets, int *sh) {
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
    w.ctr[kCtrVtChunks] = 0;
  }
  __threadfence_block();
  __syncthreads();
  // tile i of request r is emitted at E = (tiles of any request with index > i)
  // + (requests before r that also have a tile i): descending tile index first,
  // so the longest causal ranges start first.
  const int tr = a.tile_rows;
  auto place = [&](int f, int &E, int &q0, int &nq, int &r) {
    r = upper_index(tpre, nr + 1, f);
    const int i = f - tpre[r];
    E = 0;
    for (int q = 0; q < nr; ++q) {
      const int t = ntile[q];
      E += t - 1 - i > 0 ? t - 1 - i : 0;
      if (q < r && t > i) ++E;
    }
    const int c = w.sel_cnt[r];
    q0 = sel_offsets[r] + i * tr;
    nq = c - i * tr < tr ? c - i * tr : tr;
  };
  auto put = [&](int E, int q0, int nq, int r) {
    w.tiles[3 * E + 0] = q0;
    w.tiles[3 * E + 1] = nq;
    w.tiles[3 * E + 2] = r;
  };
  const int wmax = 256 / a.nkv;
  if (tcarry >= wmax) {
    for (int f = tid; f < tcarry; f += 1024) {
      int E, q0, nq, r;
      place(f, E, q0, nq, r);
      put(E, q0, nq, r);
    }
    return;
  }
  // An under-filled launch (fewer tiles than one work-group per CU, 256 CUs, for
  // each KV head) is evened out. A tile's key blocks run from its request's first
  // row, rounded down to a block, to its last query. Let H be the number of tiles
  // longer than 1.15 times a CU's share of all key blocks, at most the room left:
  // the first H tiles in emission order (the longest) each become two tiles of
  // half their queries (the second empty for a one-row tile), in their place.
  // (Thirds ran no faster than halves: with fewer queries a work-group's time per
  // key block stops falling.)
  const int f = tid;
  int E = 0, q0 = 0, nq = 0, r = 0, nb = 0;
  if (f < tcarry) {
    place(f, E, q0, nq, r);
    const int *roff = a.listed ? w.roff : a.req_offsets;
    const int last = w.tsel_row[roff[r] + (q0 - sel_offsets[r]) + nq - 1];
    nb = (last + 1 - (a.req_offsets[r] & ~(kAttnBK - 1)) + kAttnBK - 1) / kAttnBK;
  }
  int total, longer;
  block_excl_scan(nb, sh, &total);
  const long long thr = (long long)total * a.nkv * 115 / (256 * 100);
  block_excl_scan(f < tcarry && nb > thr ? 1 : 0, sh, &longer);
  const int room = min(wmax - tcarry, kAttnExtraTiles);
  const int H = min(longer, room > 0 ? room : 0);
  if (f < tcarry) {
    const int P = E + (E < H ? E : H);
    if (E < H) {
      const int h1 = (nq + 1) / 2;
      put(P, q0, h1, r);
      put(P + 1, q0 + h1, nq - h1, r);
    } else {
      put(P, q0, nq, r);
    }
  }
  if (tid == 0) w.ctr[kCtrTiles] = tcarry + H;
}

// ------------------------------------------------------------------------- //
// selection with the request resident in LDS (requests of up to kLdsEntries
// entries): keys and flags are loaded once; after marking, the key storage holds
// the grouping sequence as 16-bit entry offsets and prefix counts
// ------------------------------------------------------------------------- //
__device__ __forceinline__ int radix_digit_pass(const uint32_t *keys, const uint8_t *fl, int n,
                                                uint8_t in_bit, uint32_t prefix, uint32_t pmask,
                                                int shift, int nb, int need, int *hist, int *sh,
                                                int *digit_info, int *above_out) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const uint32_t dmask = (uint32_t)nb - 1u;
  for (int b = tid; b < nb; b += nt) hist[b] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += nt) {
    if (!(fl[i] & in_bit)) continue;
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

// Block-wide min and max of uint32 values (every thread gets both); sa and sb hold
// one int per wave.
__device__ __forceinline__ void block_minmax(uint32_t &mn, uint32_t &mx, int *sa, int *sb) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t a = (uint32_t)__shfl_xor((int)mn, o), b = (uint32_t)__shfl_xor((int)mx, o);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if (lane == 0) {
    sa[wid] = (int)mn;
    sb[wid] = (int)mx;
  }
  __syncthreads();
  for (int q = 0; q < nw; ++q) {
    const uint32_t a = (uint32_t)sa[q], b = (uint32_t)sb[q];
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  __syncthreads();
}

// Marks out_bit on the k entries with the largest keys among the n_in entries
// flagged in_bit: an MSB-first radix select finds the k-th largest key; larger keys
// are taken, and equal keys in entry order. The bits above the highest one in which
// the smallest and largest key differ are common to every key, so the digits (12,
// 12, then the rest) start below them: keys that cluster in a few exponents still
// spread over the histogram instead of piling onto a few contended bins.
__device__ void lds_mark_top(const uint32_t *keys, uint8_t *fl, int n, uint8_t in_bit,
                             uint8_t out_bit, int k, int n_in, int *hist, int *sh,
                             int *digit_info) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (k >= n_in) {
    for (int i = tid; i < n; i += nt)
      if (fl[i] & in_bit) fl[i] |= out_bit;
  } else if (k > 0) {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    for (int i = tid; i < n; i += nt)
      if (fl[i] & in_bit) {
        kmin = keys[i] < kmin ? keys[i] : kmin;
        kmax = keys[i] > kmax ? keys[i] : kmax;
      }
    block_minmax(kmin, kmax, hist, hist + 32);
    const uint32_t diff = kmin ^ kmax;
    int rem = diff ? 32 - __clz(diff) : 0;  // low bits still undecided
    uint32_t pmask = rem == 32 ? 0u : ~((1u << rem) - 1u);
    uint32_t prefix = kmin & pmask;
    int need = k;
    while (rem > 0) {
      const int width = rem < 12 ? rem : 12;
      const int shift = rem - width;
      int above;
      const int d = radix_digit_pass(keys, fl, n, in_bit, prefix, pmask, shift, 1 << width, need,
                                     hist, sh, digit_info, &above);
      need -= above;
      prefix |= (uint32_t)d << shift;
      pmask |= ((1u << width) - 1u) << shift;
      rem = shift;
    }
    int my_eq = 0;
    for (int i = tid; i < n; i += nt) {
      if (!(fl[i] & in_bit)) continue;
      if (keys[i] > prefix) fl[i] |= out_bit;
      else if (keys[i] == prefix) ++my_eq;
    }
    const int eq_tot = block_sum(my_eq, sh);
    if (eq_tot == need) {
      for (int i = tid; i < n; i += nt)
        if ((fl[i] & in_bit) && keys[i] == prefix) fl[i] |= out_bit;
    } else {
      // several equal keys at the threshold: the first `need` in entry order
      int lo, hi;
      my_segment(n, lo, hi);
      int c = 0;
      for (int i = lo; i < hi; ++i) c += ((fl[i] & in_bit) && keys[i] == prefix) ? 1 : 0;
      int t;
      int rank = block_excl_scan(c, sh, &t);
      for (int i = lo; i < hi; ++i)
        if ((fl[i] & in_bit) && keys[i] == prefix) {
          if (rank < need) fl[i] |= out_bit;
          ++rank;
        }
    }
  }
  __syncthreads();
}

// The same top-k marking with this thread's keys in registers: kr[j] is the key
// and fr[j] the flag byte of entry tid + j * blockDim.x, and bit j of cmask says
// whether that entry is flagged in_bit. Minimum, maximum and histograms read no
// LDS, and the marks of keys above the threshold's bin are plain flag stores.
// Radix passes stop once at most kRankMax keys share the decided prefix: those
// are gathered and ranked directly (larger keys, then equal keys at lower
// entries); when every bit is decided, equal keys are taken in entry order.
constexpr int kRankMax = 256;
template <int PER>
__device__ void reg_mark_top(const uint32_t (&kr)[PER], const uint8_t (&fr)[PER], uint32_t cmask,
                             const uint32_t *keys, uint8_t *fl, int n, uint8_t in_bit, uint8_t out_bit,
                             int k, int n_in, int *hist, int *sh, int *digit_info) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint32_t tmask = 0;  // entries this thread marks with a plain store at the end
  if (k >= n_in) {
    tmask = cmask;
  } else if (k > 0) {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (cmask >> j & 1u) {
        kmin = kr[j] < kmin ? kr[j] : kmin;
        kmax = kr[j] > kmax ? kr[j] : kmax;
      }
    block_minmax(kmin, kmax, hist, hist + 32);
    const uint32_t diff = kmin ^ kmax;
    int rem = diff ? 32 - __clz(diff) : 0;
    uint32_t pmask = rem == 32 ? 0u : ~((1u << rem) - 1u);
    uint32_t prefix = kmin & pmask;
    int need = k;
    int in_bin = n_in;  // keys that share the prefix decided so far
    while (rem > 0 && in_bin > kRankMax) {
      const int width = rem < 12 ? rem : 12;
      const int shift = rem - width;
      const int nb = 1 << width;
      const uint32_t dmask = (uint32_t)nb - 1u;
      for (int b = tid; b < nb; b += nt) hist[b] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if ((cmask >> j & 1u) && (kr[j] & pmask) == prefix) atomicAdd(&hist[(kr[j] >> shift) & dmask], 1);
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
        int abv = above, dsel = 0, cnt = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (abv + c[q] >= need) { dsel = nb - 1 - 4 * tid - q; cnt = c[q]; break; }
          abv += c[q];
        }
        digit_info[0] = dsel;
        digit_info[1] = abv;
        digit_info[2] = cnt;
      }
      __syncthreads();
      need -= digit_info[1];
      in_bin = digit_info[2];
      prefix |= (uint32_t)digit_info[0] << shift;
      pmask |= dmask << shift;
      rem = shift;
      __syncthreads();
    }
    // keys above the prefix's bin are taken
#pragma unroll
    for (int j = 0; j < PER; ++j)
      tmask |= ((cmask >> j & 1u) && (kr[j] & pmask) > prefix) ? 1u << j : 0u;
    if (rem == 0) {
      // the prefix is the whole key: the first `need` equal keys in entry order
      uint32_t eq = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) eq |= ((cmask >> j & 1u) && kr[j] == prefix) ? 1u << j : 0u;
      const int eq_tot = block_sum(__popc(eq), sh);
      if (eq_tot == need) {
        tmask |= eq;
      } else {
        int lo, hi;
        my_segment(n, lo, hi);
        int c = 0;
        for (int i = lo; i < hi; ++i) c += ((fl[i] & in_bit) && keys[i] == prefix) ? 1 : 0;
        int t;
        int rank = block_excl_scan(c, sh, &t);
        for (int i = lo; i < hi; ++i)
          if ((fl[i] & in_bit) && keys[i] == prefix) {
            if (rank < need) fl[i] |= out_bit;
            ++rank;
          }
      }
    } else {
      // at most kRankMax keys share the prefix: gather them as (key, ~entry) pairs,
      // whose order as 64-bit values is the selection order, and count for each
      // the larger ones, four threads per key
      uint64_t *bk = reinterpret_cast<uint64_t *>(hist);
      int *bcnt = hist + 2 * kRankMax;
      if (tid == 0) *bcnt = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if ((cmask >> j & 1u) && (kr[j] & pmask) == prefix)
          bk[atomicAdd(bcnt, 1)] = ((uint64_t)kr[j] << 32) | (uint32_t)~(uint32_t)(tid + j * nt);
      __syncthreads();
      const int nbin = *bcnt;
      const int me = tid >> 2, part = tid & 3;
      int rank = 0;
      uint64_t mine = 0;
      if (me < nbin) {
        mine = bk[me];
        for (int q = part; q < nbin; q += 16) {
          uint64_t o[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) o[u] = q + 4 * u < nbin ? bk[q + 4 * u] : 0;
#pragma unroll
          for (int u = 0; u < 4; ++u) rank += o[u] > mine ? 1 : 0;
        }
      }
      rank += __shfl_xor(rank, 1);
      rank += __shfl_xor(rank, 2);
      if (me < nbin && part == 0 && rank < need) fl[~(uint32_t)mine] |= out_bit;
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (tmask >> j & 1u) fl[tid + j * nt] = fr[j] | out_bit;
  __syncthreads();
}

// Inclusive max-scan over the wave with DPP lane shifts (INT_MIN fills lanes
// without a source, the identity of max).
__device__ __forceinline__ int wave_incl_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}

// Max over the values of the threads before this one (INT_MIN for thread 0).
// `sh` needs 17 ints of LDS.
__device__ __forceinline__ int block_excl_max(int v, int *sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int inc = wave_incl_max(v);
  const int up = __shfl_up(inc, 1, 64);
  if (lane == 63) sh[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    // wave 0: exclusive max over the wave totals
    const int t = lane < nw ? sh[lane] : INT_MIN;
    const int ti = wave_incl_max(t);
    if (lane < nw) sh[lane + 1] = ti;
    if (lane == 0) sh[0] = INT_MIN;
  }
  __syncthreads();
  const int res = max(sh[wid], lane > 0 ? up : INT_MIN);
  __syncthreads();
  return res;
}

// Sliding-window grouping over the sequence of kCand entries in order: a window of
// `win` slots starting on a kTop slot that holds at least `tau` kTop slots marks
// each of its slots kSel. seq16 (2 * kLdsEntries u16) holds slot -> entry and the
// inclusive kTop count per slot; sq (a byte per slot) is scratch.
__device__ void lds_window_group(uint8_t *fl, int n, int win, int tau, uint16_t *seq16,
                                 uint8_t *sq, int *sh) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint16_t *seq_ent = seq16;                // [n] slot -> entry offset
  uint16_t *seq_pre = seq16 + kLdsEntries;  // [n] inclusive top count
  int lo, hi;
  my_segment(n, lo, hi);
  int c = 0, tp = 0;
  for (int i = lo; i < hi; ++i)
    if (fl[i] & kCand) { ++c; tp += (fl[i] & kTop) ? 1 : 0; }
  int n_seq, n_top;
  int slot = block_excl_scan(c, sh, &n_seq);
  int run = block_excl_scan(tp, sh, &n_top);
  for (int i = lo; i < hi; ++i) {
    const uint8_t f = fl[i];
    if (!(f & kCand)) continue;
    const int top = (f & kTop) ? 1 : 0;
    run += top;
    seq_ent[slot] = (uint16_t)i;
    seq_pre[slot] = (uint16_t)run;
    sq[slot] = (uint8_t)top;
    ++slot;
  }
  __syncthreads();
  for (int t = tid; t < n_seq; t += nt) {
    if ((sq[t] & 1) && t + win <= n_seq) {
      const int cnt = (int)seq_pre[t + win - 1] - (t > 0 ? (int)seq_pre[t - 1] : 0);
      if (cnt >= tau) sq[t] |= 2;
    }
  }
  __syncthreads();
  // a slot is kept when the latest passing window start at or before it lies
  // within the window: a max-scan of passing starts over contiguous segments
  int lo2, hi2;
  my_segment(n_seq, lo2, hi2);
  int last = -1;
  for (int t = lo2; t < hi2; ++t) last = (sq[t] & 2) ? t : last;
  int rs = max(block_excl_max(last, sh), -1);
  for (int t = lo2; t < hi2; ++t) {
    if (sq[t] & 2) rs = t;
    if (rs >= 0 && rs > t - win) fl[seq_ent[t]] |= kSel;
  }
  __syncthreads();
}

__global__ __launch_bounds__(1024) void select_lds_kernel(SelectArgs a, Workspace w, int32_t *sel_offsets) {
  __shared__ int sh[17];
  __shared__ __align__(16) int hist[kHistBins];  // also the gathered (key, entry) pairs of the ranking
  __shared__ int digit_info[3];
  __shared__ uint32_t keys_s[kLdsEntries];  // later: seq_ent (u16) | seq_pre (u16)
  __shared__ uint8_t fl_s[kLdsEntries];
  __shared__ uint8_t sq_s[kLdsEntries];      // grouping: bit 0 top-k slot, bit 1 passing window
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int *roff = a.listed ? w.roff : a.req_offsets;
  const int e0 = roff[r], e1 = roff[r + 1], n = e1 - e0;

  // entry tid + j * nt of the request: flags to LDS, keys to LDS and registers
  constexpr int PER = (kLdsEntries + 1023) / 1024;
  uint32_t kr[PER];
  uint8_t fr[PER];
  uint32_t cmask = 0;
  int my_cand = 0;
  // every global load first (the LDS stores below could alias them as far as the
  // compiler knows, which would make each load wait for the previous store)
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + j * nt;
    fr[j] = i < n ? w.eflag[e0 + i] : 0;
    kr[j] = i < n ? w.keys[e0 + i] : 0u;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + j * nt;
    const uint8_t f = fr[j];
    const uint32_t key = kr[j];
    const bool cand = (f & kCand) != 0;
    fr[j] = f;
    kr[j] = cand ? key : 0u;
    cmask |= (cand ? 1u : 0u) << j;
    my_cand += cand ? 1 : 0;
    if (i < n) {
      fl_s[i] = f;
      keys_s[i] = kr[j];
    }
  }
  int my_ctx = 0;
  if (a.listed) {
    for (int j = a.req_offsets[r] + tid; j < a.req_offsets[r + 1]; j += nt) my_ctx += w.row_delta[j] != kFresh;
  } else {
    my_ctx = my_cand;  // every cached row of the request is a candidate
  }
  const int n_cand = block_sum(my_cand, sh);
  const int n_ctx = block_sum(my_ctx, sh);

  const int k = a.mode == SRP_SEL_GIVEN ? n_cand : k_from_ratio(a.ratio, n_ctx, n_cand, a.k_ceil);
  __syncthreads();  // flags and keys in LDS (the tie fallback and the grouping read them)
  reg_mark_top<PER>(kr, fr, cmask, keys_s, fl_s, n, kCand, kTop, k, n_cand, hist, sh, digit_info);

  if (a.window > 0)
    lds_window_group(fl_s, n, a.window, a.tau, reinterpret_cast<uint16_t *>(keys_s), sq_s, sh);

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
      w.tsel_row[e0 + p] = a.listed ? w.rlist[e] : e;
      w.tsel_ent[e0 + p] = e;
      ++p;
    }
  }
  if (tid == 0) w.sel_cnt[r] = total;
  if (sel_offsets) {
    // a single request: this work-group also finalizes the batch
    __threadfence_block();
    __syncthreads();
    finalize_body(a, w, sel_offsets, sh);
  }
}

// ------------------------------------------------------------------------- //
// selection by external scores (one work-group per request, resident in LDS),
// run before any projection: the chosen rows become the candidate marks of the
// R list, which the rest of the layer treats as a given list
// ------------------------------------------------------------------------- //
constexpr uint8_t kBrk = 16;    // spans: the candidate starts a run (does not join its predecessor)
constexpr uint8_t kSpan0 = 32;  // spans: a span starts at this entry
constexpr uint8_t kCap = 64;    // budget cap: kept

// Order-preserving map of a finite float onto uint32 (-0 is taken as +0), and back.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Min-max normalised score, in double as written: (s - min) / (max - min).
__device__ __forceinline__ double norm_score(uint32_t key, double mn, double range) {
#pragma clang fp contract(off)
  return ((double)key_score(key) - mn) / range;
}

// Candidate j joins the span of its predecessor i while the relative change
// |s~_j - s~_i| / s~_i stays below tau (double; a NaN or infinite change does not).
__device__ __forceinline__ bool joins(double ti, double tj, double tau) {
#pragma clang fp contract(off)
  const double delta = fabs(tj - ti) / ti;
  return delta < tau;
}

constexpr int kSegMax = (kLdsEntries + 1023) / 1024;  // entries per thread at most

// Span completion over the sequence of kCand entries in order, T_init = kTop. Every
// thread holds its contiguous share of entries in registers: a candidate either
// joins its predecessor or starts a run; runs are cut into spans of span_max slots
// from their start; each candidate adds (its kTop, 1) to a counter at its span's
// first entry (LDS atomics into ctr, which aliases the key storage), and a span
// whose kTop share reaches tau_cover marks every candidate kSel (others mark their
// kTop candidates). Returns the kSel count. sa, sb: 16 ints of scratch each.
__device__ int lds_span_complete(uint32_t *keys, uint8_t *fl, int n, int span_max, double tau_smooth,
                                 double tau_cover, int *sa, int *sb, int *sh) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;  // <= kSegMax
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  uint8_t f[kSegMax];
  uint32_t kk[kSegMax];
#pragma unroll
  for (int u = 0; u < kSegMax; ++u) {
    const bool in = lo + u < hi;
    f[u] = in ? fl[lo + u] : (uint8_t)0;
    kk[u] = in ? keys[lo + u] : 0u;
  }
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  int cnt = 0, last = -1;
#pragma unroll
  for (int u = 0; u < kSegMax; ++u)
    if (f[u] & kCand) {
      kmin = kk[u] < kmin ? kk[u] : kmin;
      kmax = kk[u] > kmax ? kk[u] : kmax;
      ++cnt;
      last = lo + u;
    }
  block_minmax(kmin, kmax, sa, sb);
  const double mn = (double)key_score(kmin);
  const double range = (double)key_score(kmax) - mn;

  // the last candidate before this share
  const int prev_last = max(block_excl_max(last, sh), -1);

  // joins (kBrk marks a candidate that starts a run) and the last run start
  int slot0, n_seq;
  slot0 = block_excl_scan(cnt, sh, &n_seq);
  int run_last = -1;
  {
    bool has_prev = prev_last >= 0;
    double tp = has_prev ? norm_score(keys[prev_last], mn, range) : 0.0;
    int slot = slot0;
#pragma unroll
    for (int u = 0; u < kSegMax; ++u) {
      if (!(f[u] & kCand)) continue;
      const double tu = norm_score(kk[u], mn, range);
      if (!(has_prev && joins(tp, tu, tau_smooth))) {
        f[u] |= kBrk;
        run_last = slot;
      }
      has_prev = true;
      tp = tu;
      ++slot;
    }
  }
  __syncthreads();  // every read of the keys is done: the storage becomes counters
  uint32_t *ctr = keys;
#pragma unroll
  for (int u = 0; u < kSegMax; ++u)
    if (lo + u < hi) ctr[lo + u] = 0u;
  const int run_in = max(block_excl_max(run_last, sh), -1);

  // span starts: every span_max slots from the run start
  int start_last = -1;
  {
    int run0 = run_in, slot = slot0;
#pragma unroll
    for (int u = 0; u < kSegMax; ++u) {
      if (!(f[u] & kCand)) continue;
      if (f[u] & kBrk) run0 = slot;
      if ((slot - run0) % span_max == 0) {
        f[u] |= kSpan0;
        start_last = lo + u;
      }
      ++slot;
    }
  }
  const int start_in = max(block_excl_max(start_last, sh), -1);

  // per-span counters: kTop count (high half) and length (low half)
  int s0e[kSegMax];
  {
    int cur = start_in;
#pragma unroll
    for (int u = 0; u < kSegMax; ++u) {
      s0e[u] = 0;
      if (!(f[u] & kCand)) continue;
      if (f[u] & kSpan0) cur = lo + u;
      s0e[u] = cur;
      atomicAdd(&ctr[cur], ((f[u] & kTop) ? 0x10000u : 0u) + 1u);
    }
  }
  __syncthreads();
  int my_sel = 0;
#pragma unroll
  for (int u = 0; u < kSegMax; ++u) {
    if (!(f[u] & kCand)) continue;
    const uint32_t v = ctr[s0e[u]];
    const bool covered = (double)(v >> 16) / (double)(v & 0xffffu) >= tau_cover;
    if (covered || (f[u] & kTop)) {
      f[u] |= kSel;
      ++my_sel;
    }
  }
#pragma unroll
  for (int u = 0; u < kSegMax; ++u)
    if (lo + u < hi) fl[lo + u] = f[u];
  const int n_sel = block_sum(my_sel, sh);
  return n_sel;
}

__global__ __launch_bounds__(1024) void score_select_kernel(SelectArgs a, Workspace w) {
  __shared__ int sh[17];
  __shared__ __align__(16) int hist[kHistBins];  // also the gathered (key, entry) pairs of the ranking
  __shared__ int digit_info[3];
  __shared__ uint32_t keys_s[kLdsEntries];  // window grouping: seq_ent (u16) | seq_pre (u16)
  __shared__ uint8_t fl_s[kLdsEntries];
  __shared__ uint8_t sq_s[kLdsEntries];
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int rq0 = a.req_offsets[r], n = a.req_offsets[r + 1] - rq0;
  // after the top-k marking the histogram storage serves as four scan arrays
  int *scan0 = hist, *scan1 = hist + 1024;

  // entry tid + j * nt of the request: flags to LDS and registers, score keys to
  // LDS and registers
  constexpr int PER = (kLdsEntries + 1023) / 1024;
  uint32_t kr[PER];
  uint8_t fr[PER];
  uint32_t cmask = 0;
  int my_ctx = 0, my_cand = 0;
  // every global load first (the LDS stores below could alias them as far as the
  // compiler knows, which would make each load wait for the previous store)
  int dlv[PER];
  uint8_t rfv[PER];
  float scv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + j * nt;
    dlv[j] = i < n ? w.row_delta[rq0 + i] : kFresh;
    rfv[j] = (i < n && a.cand) ? w.rowflag[rq0 + i] : 0;
    scv[j] = i < n ? a.scores[rq0 + i] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + j * nt;
    const int dl = dlv[j];
    const uint8_t rf = rfv[j];
    const float sc = scv[j];
    const bool fresh = dl == kFresh;
    const bool cand = i < n && !fresh && (a.cand ? rf == kCand : true);
    fr[j] = fresh ? kFreshF : (cand ? kCand : 0);
    kr[j] = cand ? score_key(sc) : 0u;
    cmask |= (cand ? 1u : 0u) << j;
    if (i < n) {
      fl_s[i] = fr[j];
      keys_s[i] = kr[j];
      my_ctx += fresh ? 0 : 1;
    }
    my_cand += cand ? 1 : 0;
  }
  const int n_ctx = block_sum(my_ctx, sh);
  const int n_cand = block_sum(my_cand, sh);

  const int k = k_from_ratio(a.ratio, n_ctx, n_cand, a.k_ceil);
  __syncthreads();  // flags and keys in LDS
  reg_mark_top<PER>(kr, fr, cmask, keys_s, fl_s, n, kCand, kTop, k, n_cand, hist, sh, digit_info);

  uint8_t chosen = kTop;
  if (a.span_max > 0) {
    const int n_sel = lds_span_complete(keys_s, fl_s, n, a.span_max, a.tau_smooth, a.tau_cover,
                                        scan0, scan1, sh);
    chosen = kSel;
    if (a.cap_ratio > 0.0) {
      const int m = k_from_ratio(a.cap_ratio, n_ctx, n_cand, a.k_ceil);
      if (n_sel > m) {
        // the key storage held the span counters: reload the keys of the chosen rows
        // (all loads before the LDS stores, as above)
        float scv[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int i = tid + j * nt;
          scv[j] = (i < n && (fl_s[i] & kSel)) ? a.scores[rq0 + i] : 0.f;
        }
        __syncthreads();  // every thread has read its flags before keys_s changes
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int i = tid + j * nt;
          if (i < n) keys_s[i] = (fl_s[i] & kSel) ? score_key(scv[j]) : 0u;
        }
        __syncthreads();
        lds_mark_top(keys_s, fl_s, n, kSel, kCap, m, n_sel, hist, sh, digit_info);
        chosen = kCap;
      }
    }
  } else if (a.window > 0) {
    lds_window_group(fl_s, n, a.window, a.tau, reinterpret_cast<uint16_t *>(keys_s), sq_s, sh);
    chosen = kSel;
  }
  __syncthreads();
  for (int i = tid; i < n; i += nt) w.rowflag[rq0 + i] = (fl_s[i] & chosen) ? kCand : 0;
  if (gridDim.x == 1) {
    // a single request: the R list (chosen rows and fresh rows in row order) right
    // here instead of three grid-wide passes
    int lo, hi;
    my_segment(n, lo, hi);
    int c = 0;
    for (int i = lo; i < hi; ++i) c += (fl_s[i] & (chosen | kFreshF)) ? 1 : 0;
    int total;
    int p = block_excl_scan(c, sh, &total);
    for (int i = lo; i < hi; ++i)
      if (fl_s[i] & (chosen | kFreshF)) w.rlist[p++] = rq0 + i;
    if (tid == 0) {
      w.roff[0] = 0;
      w.roff[1] = total;
      w.ctr[kCtrREntries] = total;
    }
  }
}

__global__ __launch_bounds__(1024) void finalize_kernel(SelectArgs a, Workspace w, int32_t *sel_offsets) {
  __shared__ int sh[17];
  finalize_body(a, w, sel_offsets, sh);
}

// ------------------------------------------------------------------------- //
// compaction to sel_idx and scatter of the fresh K/V rows (one wave per entry);
// with fresh_all every recomputed entry's fresh K/V goes to its row instead
// ------------------------------------------------------------------------- //
// Copies one row's fresh K and V (16-byte chunks, a wave per row) into cache row
// cr, two chunks per lane and operand at a time with all four loads issued before
// the stores (the compiler cannot tell the scratch from the cache, so it would
// otherwise wait on each load before the next).
template <typename T>
__device__ __forceinline__ void scatter_row(const T *f, int kvdim, bool v_only, T *k_cache, T *v_cache, int cr,
                                            int lane) {
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte chunk
  const int chunks = kvdim / V;
  T *kd = k_cache + (size_t)cr * kvdim, *vd = v_cache + (size_t)cr * kvdim;
  for (int c = lane; c < chunks; c += 128) {
    // the second chunk's loads come from a clamped (always valid) chunk
    const int c2 = min(c + 64, chunks - 1);
    uint4 k0 = {0, 0, 0, 0}, k1 = {0, 0, 0, 0};
    if (!v_only) {
      k0 = *reinterpret_cast<const uint4 *>(f + c * V);
      k1 = *reinterpret_cast<const uint4 *>(f + c2 * V);
    }
    const uint4 v0 = *reinterpret_cast<const uint4 *>(f + kvdim + c * V);
    const uint4 v1 = *reinterpret_cast<const uint4 *>(f + kvdim + c2 * V);
    if (!v_only) *reinterpret_cast<uint4 *>(kd + c * V) = k0;
    *reinterpret_cast<uint4 *>(vd + c * V) = v0;
    if (c + 64 < chunks) {
      if (!v_only) *reinterpret_cast<uint4 *>(kd + (c + 64) * V) = k1;
      *reinterpret_cast<uint4 *>(vd + (c + 64) * V) = v1;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void compact_scatter_kernel(SelectArgs a, Workspace w, int kvdim,
                                                              int32_t *sel_idx, const int32_t *sel_offsets,
                                                              T *k_cache, T *v_cache) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int *roff = a.listed ? w.roff : a.req_offsets;
  // batches of fewer than 64 requests: lane i holds the request tables' entry i,
  // so a row's request comes from one ballot, not a chain of dependent loads
  const bool lanes = a.n_req < 64;
  int ro_l = 0, so_l = 0, sc_l = 0;
  if (lanes && lane <= a.n_req) {
    ro_l = roff[lane];
    so_l = sel_offsets[lane];
    if (a.fresh_all && lane < a.n_req) sc_l = w.sel_cnt[lane];
  }
  if (!a.fresh_all) {
    // selected rows only: output slot s of request r is entry roff[r] + (s -
    // sel_offsets[r]) of the per-request selection
    const int total = lanes ? __shfl(so_l, a.n_req, 64) : sel_offsets[a.n_req];
    for (int s = wave; s < total; s += nwaves) {
      int r, q;
      if (lanes) {
        r = upper_index_lanes(so_l, a.n_req + 1, s);
        q = __shfl(ro_l, r, 64) + (s - __shfl(so_l, r, 64));
      } else {
        r = upper_index(sel_offsets, a.n_req + 1, s);
        q = roff[r] + (s - sel_offsets[r]);
      }
      const int row = w.tsel_row[q], e = w.tsel_ent[q];
      if (lane == 0) {
        sel_idx[s] = row;
        w.sel_ent[s] = e;
      }
      const T *f = (const T *)w.fresh_kv + (size_t)e * 2 * kvdim;
      const int cr = w.row_slot ? w.row_slot[row] : row;  // cache row
      scatter_row(f, kvdim, a.v_only, k_cache, v_cache, cr, lane);
    }
    return;
  }
  // fresh K/V of every recomputed row (the selected ones also fill sel_idx)
  const int nR = lanes ? __shfl(ro_l, a.n_req, 64) : roff[a.n_req];
  for (int q = wave; q < nR; q += nwaves) {
    int i, cnt, so;
    if (lanes) {
      const int r = upper_index_lanes(ro_l, a.n_req + 1, q);
      i = q - __shfl(ro_l, r, 64);
      cnt = __shfl(sc_l, r, 64);
      so = __shfl(so_l, r, 64);
    } else {
      const int r = upper_index(roff, a.n_req + 1, q);
      i = q - roff[r];
      cnt = w.sel_cnt[r];
      so = sel_offsets[r];
    }
    int row = -1, e = -1;
    if (i < cnt) {
      const int out = so + i;
      row = w.tsel_row[q];
      e = w.tsel_ent[q];
      if (lane == 0) {
        sel_idx[out] = row;
        w.sel_ent[out] = e;
      }
    }
    e = q;
    row = a.listed ? w.rlist[q] : q;
    const T *f = (const T *)w.fresh_kv + (size_t)e * 2 * kvdim;
    const int cr = w.row_slot ? w.row_slot[row] : row;  // cache row
    scatter_row(f, kvdim, a.v_only, k_cache, v_cache, cr, lane);
  }
}

// ------------------------------------------------------------------------- //
// launchers
// ------------------------------------------------------------------------- //
hipError_t launch_prepare(const SelectArgs &a, const Workspace &w, hipStream_t s) {
  if (a.cand && a.listed && a.mode != SRP_SEL_SCORES && a.T > 0 && a.T <= kPrepOneGroup) {
    hipLaunchKernelGGL(prepare_one_group_kernel, dim3(1), dim3(1024), 0, s, a, w);
    return hipGetLastError();
  }
  if (a.T > 0) {
    int grid = (a.T + 255) / 256;
    grid = grid < 4096 ? grid : 4096;
    hipLaunchKernelGGL(row_meta_kernel, dim3(grid), dim3(256), 0, s, a, w);
  }
  if (a.cand) {
    int grid = (a.T + 255) / 256;
    grid = grid < 1024 ? (grid > 0 ? grid : 1) : 1024;
    hipLaunchKernelGGL(mark_cand_kernel, dim3(grid), dim3(256), 0, s, a, w);
  }
  if (a.mode == SRP_SEL_SCORES)
    hipLaunchKernelGGL(score_select_kernel, dim3(a.n_req), dim3(1024), 0, s, a, w);
  // the external-score selection of a single request writes the R list itself
  if (a.listed && !(a.mode == SRP_SEL_SCORES && a.n_req == 1)) {
    const int bpr = blocks_per_req(a.max_req_rows);
    hipLaunchKernelGGL(r_count_kernel, dim3(a.n_req * bpr), dim3(1024), 0, s, a, w, bpr);
    hipLaunchKernelGGL(r_scan_kernel, dim3(1), dim3(1024), 0, s, a, w, bpr);
    hipLaunchKernelGGL(r_write_kernel, dim3(a.n_req * bpr), dim3(1024), 0, s, a, w, bpr);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs &a, const Workspace &w, int32_t *sel_offsets, hipStream_t s) {
  int grid = (a.T + 255) / 256;
  grid = grid < 2048 ? (grid > 0 ? grid : 1) : 2048;
  hipLaunchKernelGGL(keys_kernel, dim3(grid), dim3(256), 0, s, a, w);
  if (a.max_req_rows <= kLdsEntries) {
    // a single request's work-group finalizes the batch itself
    hipLaunchKernelGGL(select_lds_kernel, dim3(a.n_req), dim3(1024), 0, s, a, w,
                       a.n_req == 1 ? sel_offsets : nullptr);
    if (a.n_req == 1) return hipGetLastError();
  } else {
    hipLaunchKernelGGL(select_kernel, dim3(a.n_req), dim3(1024), 0, s, a, w);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, s, a, w, sel_offsets);
  return hipGetLastError();
}


hipError_t launch_compact_scatter(const SelectArgs &a, const Workspace &w, int dtype, int kvdim,
                                  int32_t *sel_idx, const int32_t *sel_offsets, void *k_cache,
                                  void *v_cache, hipStream_t s) {
  // a wave per row up to two rounds of resident waves (32 per CU), rows beyond that
  // strided over them: the selection's size is known on the device only, and at
  // small ratios a wave per cached row mostly finds no row and only adds dispatch
  // rounds (16K waves: 16 against 18 us at 5% of 128K rows, 92 against 89 us at 50%)
  int grid = (a.T * 64 + 255) / 256;
  grid = grid < 4096 ? (grid > 0 ? grid : 1) : 4096;
  if (dtype == SRP_BF16)
    hipLaunchKernelGGL(compact_scatter_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, a, w, kvdim,
                       sel_idx, sel_offsets, (uint16_t *)k_cache, (uint16_t *)v_cache);
  else
    hipLaunchKernelGGL(compact_scatter_kernel<float>, dim3(grid), dim3(256), 0, s, a, w, kvdim,
                       sel_idx, sel_offsets, (float *)k_cache, (float *)v_cache);
  return hipGetLastError();
}

}  // namespace srp
